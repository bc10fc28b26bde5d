// Warp-specialised chunkwise prefill (bf16 q/k/v, no gate or a scalar gate).
//
// Same mathematics as chunk_fwd.hip (section 6 of "You Could Have Come Up With
// Kimi Delta Attention"; section 4 of "From Attention to Learned Memory"): per
// chunk of C = 64 tokens with incoming state S (S^T resident in registers),
//
//   R  = strict-lower(beta_i (k_i . k_j) e^{G_i - G_j}),  T = (I + R)^{-1}
//   A  = lower(scale (q_i . k_j) e^{G_i - G_j})
//   Vb = T (beta (V - e^{G} (K S^T)))          (delta rule; Vb = V for the linear rule)
//   O  = scale e^{G} (Q S^T) + A Vb
//   S^T <- e^{G_last} S^T + K^T (e^{G_last - G_j} Vb_j)
//
// The work of a chunk is split between two groups of waves that run
// concurrently; a workgroup covers BVW = 16 * NSW value columns of one
// (sequence, value head):
//
//   * state waves 0 .. NSW-1 own 16 value columns each (S^T[DK, 16] in MFMA
//     accumulators) and do everything that depends on the state: the products
//     with the state, Vb, the outputs and the state update. Every product is a
//     16x16x32 MFMA, and the LDS fragments of the next step are in flight
//     while the current one multiplies;
//   * prep waves NSW .. NSW+3 do everything that does not, one chunk ahead:
//     write the next chunk's keys and queries into LDS (from registers loaded
//     one more chunk ahead), the gate prefix sums, R and A, the 16x16
//     diagonal inverses of I + R, and then the whole of T by block forward
//     substitution, one 16-column block of T per prep wave. T and A stay in
//     registers across the end-of-chunk barrier and go to LDS right after it.
//
// Keys, queries and gate factors are double buffered in LDS (set c % 2 is read
// by the state waves while the prep waves fill set (c+1) % 2). T and A are
// single buffered: the prep waves store them after the barrier that ends the
// previous chunk and count their stores on an LDS counter, on which the state
// waves wait just before their first use. One workgroup barrier per chunk.
//
// The state update reads K^T fragments straight from the token-major key
// array with the transposing LDS read of gfx950 (ds_read_b64_tr_b16).
#include <type_traits>

#include "chunk_common.h"

namespace gdr {
namespace {

using namespace chunk;

constexpr int NSTG = 4;           // prep waves that stage keys and queries (64 * NSTG threads)

// Prep waves per workgroup: six beside two state waves (then every SIMD runs
// two waves), four beside four state waves (the registers allow no more).
template <int NSW> constexpr int prep_waves() { return NSW == 2 ? 6 : 4; }

// What prep wave w (of np) does per chunk. Gram tiles come in segments:
// row block `row` of R (kind 1) or A (kind 2), tile columns j0 .. j1; R
// segments come first. The wave may invert one diagonal block of R (whose
// tile it forms), solve one block column of T, and stage keys and queries
// (stager index 0..3). With six prep waves the four on the SIMDs without a
// state wave stage, form and invert one diagonal block each and solve one
// column of T (the two long columns on different SIMDs); the two that share a
// SIMD with a state wave form the six off-diagonal tiles of R, row 1 first.
// The solves follow R row by row (a counter per row), so they overlap the
// long rows. A, which is needed only after the end-of-chunk barrier, goes to
// the waves with the shortest chains: the two with short T columns (before
// their solve) and the two R waves (after R). With four prep waves wave w
// forms row 3 - w of R, inverts its diagonal block and solves T column 3 - w
// (every row of R is waited for before any solve), and forms row w of A: the
// longest solve (column 0) falls to the wave with the shortest R row, and each
// wave forms five Gram tiles.
struct SegWS {
  int kind, row, j0, j1;
};
struct RoleWS {
  SegWS seg[4];
  int inv, tcol, stager;
};
constexpr SegWS NOSEG = {0, 0, 0, 0};
constexpr RoleWS role_ws(bool delta, int np, int w) {
  if (!delta) {
    if (np == 4) return {{{2, 3 - w, 0, 3 - w}, NOSEG, NOSEG, NOSEG}, -1, -1, w};
    switch (w) {
      case 0: return {{{2, 3, 0, 3}, NOSEG, NOSEG, NOSEG}, -1, -1, 0};
      case 1: return {{{2, 2, 0, 2}, NOSEG, NOSEG, NOSEG}, -1, -1, 1};
      case 4: return {{{2, 1, 0, 1}, NOSEG, NOSEG, NOSEG}, -1, -1, 2};
      case 5: return {{{2, 0, 0, 0}, NOSEG, NOSEG, NOSEG}, -1, -1, 3};
      default: return {{NOSEG, NOSEG, NOSEG, NOSEG}, -1, -1, -1};
    }
  }
  if (np == 4) return {{{1, 3 - w, 0, 3 - w}, {2, w, 0, w}, NOSEG, NOSEG}, 3 - w, 3 - w, w};
  switch (w) {
    case 0: return {{{1, 0, 0, 0}, {2, 0, 0, 0}, {2, 1, 0, 1}, NOSEG}, 0, 3, 0};
    case 1: return {{{1, 1, 1, 1}, {2, 2, 0, 2}, NOSEG, NOSEG}, 1, 2, 1};
    case 2: return {{{1, 1, 0, 0}, {1, 2, 0, 1}, {2, 3, 0, 1}, NOSEG}, -1, -1, -1};
    case 3: return {{{1, 3, 0, 2}, {2, 3, 2, 3}, NOSEG, NOSEG}, -1, -1, -1};
    case 4: return {{{1, 2, 2, 2}, NOSEG, NOSEG, NOSEG}, 2, 1, 2};
    default: return {{{1, 3, 3, 3}, NOSEG, NOSEG, NOSEG}, 3, 0, 3};
  }
}
// Whether an R segment counts in on its row's counter on its own: it holds
// tiles left of the diagonal and its wave does not invert that row's
// diagonal block (a wave that does counts in once, after the inverse).
constexpr bool counts_row(const RoleWS &rl, const SegWS &s) {
  return s.kind == 1 && s.j0 < s.row && rl.inv != s.row;
}
// Waves that count in on row I's counter per chunk: row I of R (left of the
// diagonal) and T_II are complete once all of them have.
constexpr int row_producers(bool delta, int np, int I) {
  int n = 0;
  for (int w = 0; w < np; ++w) {
    const RoleWS rl = role_ws(delta, np, w);
    if (rl.inv == I) ++n;
    for (int k = 0; k < 4; ++k) n += rl.seg[k].row == I && counts_row(rl, rl.seg[k]);
  }
  return n;
}


template <int D, int NSW>
struct SmemWS {
  // bf16 token-major key and query rows (permuted k blocks): a row pitch of
  // 32 bytes modulo 128 keeps the 16-byte fragment reads free of bank conflicts
  static constexpr int PK = D + 16;
  static constexpr int PT = C + 16;   // bf16 rows of T and A (permuted 32-token blocks)
  static constexpr int PR = C + 8;    // bf16 rows of R (8-byte fragment reads)
  struct alignas(16) Set {
    uint16_t kk[C][PK];
    uint16_t qq[C][PK];
    float G[C], eG[C], eGl[C], beta[C];
    float eB[C];   // e^{G_b - G_j} with G_b the gate sum at the last token of j's 16-token block (<= 1)
    float eGlast, pad_[3];
  };
  // The fixed-address arrays come first and stay within the 64 KiB that an
  // LDS instruction's immediate offset reaches, so their many access sites
  // share a few base registers; the sets are addressed from a per-chunk base.
  int kcount;   // stagers: keys and gate factors stored (4 per chunk)
  int qcount;   // stagers: queries stored (4 per chunk)
  int tcount;   // prep waves: T stored (one per prep wave and chunk)
  int acount;   // prep waves: A stored (one per prep wave and chunk)
  uint16_t th[C][PT], tl[C][PT];   // T of the chunk the state waves are on (split bf16)
  uint16_t ah[C][PT], al[C][PT];   // A of that chunk
  uint16_t rh[C][PR], rl[C][PR];   // R's off-diagonal blocks (prep waves only)
  float rd[4][16][20];             // R's diagonal blocks negated, then their inverses (prep waves only)
  uint16_t vx[NSW][C][16];         // per state wave: its value columns, token-major (swizzled halves)
  Set set[2];
  alignas(16) int rcount[4];   // row I of R and T_II done (row_producers per chunk)
};

// Prep-wave registers for one chunk's keys, queries and gates.
template <int D>
struct PrefWS {
  static constexpr int KU = C * D / 8 / (64 * NSTG);   // 16-byte units per staging thread
  typename U32Vec<4 * KU>::type k, q;
  float g, beta;
  bool gfirst;   // (more than one transition per token) the row is a token's first substep
};

// Registers a prep wave carries across the end-of-chunk barrier: its block
// column of T and its tiles of A, all in row layout (lane (r, g) holds row
// r of a 16x16 block, columns 4g .. 4g+3).
struct HoldWS {
  f32x4 tdiag;      // T_JJ
  f32x4 trow[4];    // T_IJ for I > J
  f32x4 a[2][4];    // tile J of the wave's A segment `slot`
};

// 16-byte LDS read of four floats at an address known to be that aligned.
__device__ __forceinline__ float4 ld4(const float *p) {
  return *static_cast<const float4 *>(__builtin_assume_aligned(p, 16));
}

// LDS stores of 8 and 16 bytes at addresses known to be that aligned (so
// they compile to single ds_write_b64 / ds_write_b128 instructions).
__device__ __forceinline__ void st8(void *p, uint2 v) {
  *static_cast<uint2 *>(__builtin_assume_aligned(p, 8)) = v;
}
__device__ __forceinline__ void st16(void *p, uint4 v) {
  *static_cast<uint4 *>(__builtin_assume_aligned(p, 16)) = v;
}

// Four values split into packed bf16 hi and lo (see split_pair).
__device__ __forceinline__ uint2 pack_hi(const f32x4 &x, uint2 &lo) {
  uint32_t h0, l0, h1, l1;
  split_pair(x[0], x[1], h0, l0);
  split_pair(x[2], x[3], h1, l1);
  lo = make_uint2(l0, l1);
  return make_uint2(h0, h1);
}

// 16x16x32 A fragment of a split bf16 plane pair: row `row`, k step `s`.
__device__ __forceinline__ void ldfrag2(const uint16_t *hi, const uint16_t *lo, int pitch, int row,
                                        int s, int g, Frag &f) {
  const int o = row * pitch + 32 * s + 8 * g;
  f.hi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(hi + o));
  f.lo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(lo + o));
}

// Rows t0 .. t0 + L - 1 of a chunk (clamped to the last). With PROD (P > 1
// transitions per token) the rows are substeps: keys and beta by substep,
// the query of the substep's token (only a token's last substep keeps its
// output, and an output row depends on no other row's query), and the
// token's gate on its first substep only (gfirst; the others decay by 1).
// With REV the sequence is walked backwards: its row t is memory row
// mirror - t (mirror = the sequence's first row + its last row).
template <int GATE, bool DELTA, int D, bool PROD, bool REV>
__device__ __forceinline__ void prep_load(PrefWS<D> &pf, const ChunkParams &p, int64_t t0, int L,
                                          int h, int hk, int ptid, int64_t mirror) {
  constexpr int KU = PrefWS<D>::KU;
  const int krow = ptid / (D / 8), krs = 64 * NSTG / (D / 8), kc = (ptid % (D / 8)) * 16;
  const char *kb = static_cast<const char *>(p.k) + (t0 * p.k_stride + (int64_t)hk * D) * 2;
  const char *qb = static_cast<const char *>(p.q) + ((PROD ? t0 / p.P : t0) * p.q_stride + (int64_t)hk * D) * 2;
  const uint32_t ks = (uint32_t)(p.k_stride * 2), qs = (uint32_t)(p.q_stride * 2);
  const int last = L - 1;
  if constexpr (REV) {
    // the chunk's rows t0 .. t0 + last are memory rows bot + last .. bot:
    // 32-bit offsets up from the lowest, as in the forward walk
    const int64_t bot = mirror - t0 - last;
    const char *kl = static_cast<const char *>(p.k) + (bot * p.k_stride + (int64_t)hk * D) * 2;
    const char *ql = static_cast<const char *>(p.q) + (bot * p.q_stride + (int64_t)hk * D) * 2;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t up = (uint32_t)(last - min(krow + u * krs, last));
      put4(pf.k, u, *reinterpret_cast<const uint4 *>(kl + (up * ks + kc)));
      put4(pf.q, u, *reinterpret_cast<const uint4 *>(ql + (up * qs + kc)));
    }
    if (ptid < 64) {
      const int64_t th = (bot + last - min(ptid, last)) * p.HV + h;
      if constexpr (GATE == GDR_GATE_SCALAR) pf.g = p.g[th];
      if constexpr (DELTA) pf.beta = p.beta[th];
    }
  } else if constexpr (!PROD) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t row = (uint32_t)min(krow + u * krs, last);
      put4(pf.k, u, *reinterpret_cast<const uint4 *>(kb + (row * ks + kc)));
      put4(pf.q, u, *reinterpret_cast<const uint4 *>(qb + (row * qs + kc)));
    }
    if (ptid < 64) {
      const int64_t th = (t0 + min(ptid, last)) * p.HV + h;
      if constexpr (GATE == GDR_GATE_SCALAR) pf.g = p.g[th];
      if constexpr (DELTA) pf.beta = p.beta[th];
    }
  } else {
    const SubMap sm_(t0, p.P);   // qb starts at its token r0
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t row = (uint32_t)min(krow + u * krs, last);
      const uint32_t qr = (uint32_t)sm_.tok((int)row);
      put4(pf.k, u, *reinterpret_cast<const uint4 *>(kb + (row * ks + kc)));
      put4(pf.q, u, *reinterpret_cast<const uint4 *>(qb + (qr * qs + kc)));
    }
    if (ptid < 64) {
      const int row = min(ptid, last);
      if constexpr (GATE == GDR_GATE_SCALAR) pf.g = p.g[(sm_.r0 + sm_.tok(row)) * p.HV + h];
      pf.gfirst = sm_.sub(row) == 0;
      if constexpr (DELTA) pf.beta = p.beta[(t0 + row) * p.HV + h];
    }
  }
}

// One segment of Gram tiles: row block I of R (KIND 1) or A (KIND 2), tile
// columns J0 .. J1. Tile (I, J) is computed transposed (keys of block J as
// the M operand), so a lane ends with row ii = 16I + r, columns
// 16J + 4g .. +3. R's off-diagonal tiles go to the R planes, its diagonal
// tile negated in fp32 to rd; A's tiles stay in registers (h.a[SLOT]).
template <int KIND, int I, int J0, int J1, int SLOT, int GATE, int D, class SM>
__device__ __forceinline__ void gram_seg(SM &sm, const typename SM::Set &S, float scale, int r, int g,
                                         HoldWS &h) {
  constexpr int NS = D / 32;
  constexpr int PK = SM::PK;
  constexpr bool ISA = KIND == 2;
  Frag fn[NS], fm[2][NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ldfrag(ISA ? &S.qq[0][0] : &S.kk[0][0], PK, 16 * I + r, 32 * s, g, fn[s]);
    ldfrag(&S.kk[0][0], PK, 16 * J0 + r, 32 * s, g, fm[0][s]);
  }
  f32x4 acc[J1 + 1];
#pragma unroll
  for (int J = J0; J <= J1; ++J) {
    if (J < J1) {
#pragma unroll
      for (int s = 0; s < NS; ++s) ldfrag(&S.kk[0][0], PK, 16 * (J + 1) + r, 32 * s, g, fm[(J + 1 - J0) & 1][s]);
    }
    __builtin_amdgcn_sched_barrier(0);
    // even and odd k steps in two accumulators, so consecutive MFMAs are
    // independent
    f32x4 a2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int s = 0; s < NS; ++s) a2[s & 1] = mfma(fm[(J - J0) & 1][s].hi, fn[s].hi, a2[s & 1]);
    acc[J] = a2[0] + a2[1];
    __builtin_amdgcn_sched_barrier(0);
  }
  const int ii = 16 * I + r;
  const float Gi = S.G[ii], coef = ISA ? scale : S.beta[ii];
#pragma unroll
  for (int J = J0; J <= J1; ++J) {
    // decay e^{G_i - G_j}: on a diagonal tile directly (and the causal
    // mask); below it, as e^{G_i - G_b} e^{G_b - G_j} with G_b the gate sum
    // at block J's last token, both factors <= 1 (G never increases)
    f32x4 gam = {1.f, 1.f, 1.f, 1.f};
    if constexpr (GATE == GDR_GATE_SCALAR) {
      if (J == I) {
        const float4 Gj4 = *reinterpret_cast<const float4 *>(&S.G[16 * J + 4 * g]);
        gam = f32x4{__expf(Gi - Gj4.x), __expf(Gi - Gj4.y), __expf(Gi - Gj4.z), __expf(Gi - Gj4.w)};
      } else {
        const float a = __expf(Gi - S.G[16 * J + 15]);
        const float4 b4 = *reinterpret_cast<const float4 *>(&S.eB[16 * J + 4 * g]);
        gam = f32x4{a * b4.x, a * b4.y, a * b4.z, a * b4.w};
      }
    }
    f32x4 val;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jj = 16 * J + 4 * g + i;
      val[i] = coef * acc[J][i] * gam[i];
      if (J == I) val[i] = (ISA ? jj <= ii : jj < ii) ? val[i] : 0.f;
    }
    if constexpr (ISA) {
      h.a[SLOT][J] = val;
    } else if (J == I) {
      // stored negated, the form the in-register inverse takes
      *reinterpret_cast<float4 *>(&sm.rd[I][r][4 * g]) = make_float4(-val[0], -val[1], -val[2], -val[3]);
    } else {
      uint2 lo;
      const uint2 hi = pack_hi(val, lo);
      st8(&sm.rh[ii][16 * J + 4 * g], hi);
      st8(&sm.rl[ii][16 * J + 4 * g], lo);
    }
  }
}

// T_II = (I + R_II)^{-1} in place in rd[I]: lane (r, g) reads row r of
// -R_II (written by lanes (r, 0..3) of this wave), inverts in registers,
// writes back its four entries of row r of T_II.
template <int I, class SM>
__device__ __forceinline__ void invert_diag(SM &sm, int r, int g) {
  float nrow16[16], t[4];   // row r of -R_II; row r, columns 4g .. 4g+3 of T_II
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    const float4 v4 = *reinterpret_cast<const float4 *>(&sm.rd[I][r][4 * i4]);
    nrow16[4 * i4] = v4.x; nrow16[4 * i4 + 1] = v4.y; nrow16[4 * i4 + 2] = v4.z; nrow16[4 * i4 + 3] = v4.w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = (r == 4 * g + i) ? 1.f : 0.f;
  unit_lower_inverse16(t, nrow16);
  *reinterpret_cast<float4 *>(&sm.rd[I][r][4 * g]) = make_float4(t[0], t[1], t[2], t[3]);
}

// All segments of prep wave W's role of kind KIND, in order (A segments take
// hold slots 0, 1 in order).
template <int KIND, int W, int NP, int GATE, bool DELTA, int D, class SM>
__device__ __forceinline__ void gram_role(SM &sm, const typename SM::Set &S, float scale, int r, int g,
                                          int lane, HoldWS &h) {
  constexpr RoleWS RL = role_ws(DELTA, NP, W);
  constexpr SegWS S0 = RL.seg[0], S1 = RL.seg[1], S2 = RL.seg[2], S3 = RL.seg[3];
  constexpr int SL1 = S0.kind == 2 ? 1 : 0;
  constexpr int SL2 = SL1 + (S1.kind == 2 ? 1 : 0);
  constexpr int SL3 = SL2 + (S2.kind == 2 ? 1 : 0);
  if constexpr (S0.kind == KIND) {
    gram_seg<KIND, S0.row, S0.j0, S0.j1, 0, GATE, D>(sm, S, scale, r, g, h);
    if constexpr (counts_row(RL, S0)) count_in(&sm.rcount[S0.row], lane);
  }
  if constexpr (S1.kind == KIND) {
    gram_seg<KIND, S1.row, S1.j0, S1.j1, SL1, GATE, D>(sm, S, scale, r, g, h);
    if constexpr (counts_row(RL, S1)) count_in(&sm.rcount[S1.row], lane);
  }
  if constexpr (S2.kind == KIND) {
    gram_seg<KIND, S2.row, S2.j0, S2.j1, SL2, GATE, D>(sm, S, scale, r, g, h);
    if constexpr (counts_row(RL, S2)) count_in(&sm.rcount[S2.row], lane);
  }
  if constexpr (S3.kind == KIND) {
    gram_seg<KIND, S3.row, S3.j0, S3.j1, SL3, GATE, D>(sm, S, scale, r, g, h);
    if constexpr (counts_row(RL, S3)) count_in(&sm.rcount[S3.row], lane);
  }
}

// Block column J of T = (I + R)^{-1} by forward substitution over 16-row
// blocks: T_JJ from rd, then for I > J
//     T_IJ = -T_II (sum_{K=J}^{I-1} R_IK T_KJ)
// (16x16x16 products; R_IK and T_II in row layout as A operands, T_KJ in
// accumulator layout, which is the B operand layout). Each T_IJ is also
// formed transposed, (T_II acc)^T = acc^T T_II^T, with the same registers
// as swapped operands: that product comes out in row layout, for the store.
// With six prep waves, block row I starts once its counter says row I of R
// and T_II are done, so the solve overlaps the forming of the rows below
// (the long rows are formed by other waves); with four, each wave forms a
// whole row and all rows are waited for up front, which keeps the loads of
// the solve free to run ahead.
template <int J, int NP, class SM>
__device__ __forceinline__ void solve_col(const SM &sm, int r, int g, HoldWS &h, int ci) {
  constexpr int PR = SM::PR;
  constexpr bool PER_ROW = NP > 4;
  if constexpr (PER_ROW) {
    spin_until(&sm.rcount[J], row_producers(true, NP, J) * (ci + 1));
  } else {
    // all four row counters in one 16-byte read per poll
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) volatile i32x4 lds_vi32x4;
    const lds_vi32x4 *q = (const lds_vi32x4 *)&sm.rcount[0];
    bool done = false;
    for (int spin = 0; spin < SPIN; ++spin) {
      const i32x4 v = *q;
      const int n = ci + 1;
      if ((J > 0 || v[0] >= row_producers(true, NP, 0) * n) && (J > 1 || v[1] >= row_producers(true, NP, 1) * n) &&
          (J > 2 || v[2] >= row_producers(true, NP, 2) * n) && v[3] >= row_producers(true, NP, 3) * n) {
        done = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!done) note_wait_timeout();
    asm volatile("" ::: "memory");
  }
  {
    const float4 d = *reinterpret_cast<const float4 *>(&sm.rd[J][r][4 * g]);
    h.tdiag = f32x4{d.x, d.y, d.z, d.w};
  }
  Frag4 tcol[4];
  {
    f32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = sm.rd[J][4 * g + i][r];   // column r of T_JJ
    split4(c, tcol[J]);
  }
#pragma unroll
  for (int I = J + 1; I < 4; ++I) {
    // row I of R and T_II of this chunk are complete
    if constexpr (PER_ROW) spin_until(&sm.rcount[I], row_producers(true, NP, I) * (ci + 1));
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int K = J; K < I; ++K) {
      Frag4 fr;
      ldsplit4(&sm.rh[0][0], &sm.rl[0][0], PR, 16 * I + r, 16 * K, g, fr);
      acc = mm16(fr, tcol[K], acc);
    }
    Frag4 ft, fy;
    const float4 d = *reinterpret_cast<const float4 *>(&sm.rd[I][r][4 * g]);
    split4(f32x4{d.x, d.y, d.z, d.w}, ft);
    split4(acc, fy);
    h.trow[I] = -mm16(fy, ft, f32x4{0.f, 0.f, 0.f, 0.f});
    if (I < 3) split4(-mm16(ft, fy, f32x4{0.f, 0.f, 0.f, 0.f}), tcol[I]);
  }
}

// Store a prep wave's T block column (STORE_T) or its A tiles (held across
// the barrier) into the single-buffered planes: row-major, token columns of
// each 32-block permuted (perm32) so that a state wave's fragment is one
// 16-byte read.
template <int W, int NP, bool DELTA, bool STORE_T, class SM>
__device__ __forceinline__ void store_hold(SM &sm, const HoldWS &h, int r, int g) {
  constexpr int PT = SM::PT;
  constexpr RoleWS RL = role_ws(DELTA, NP, W);
  auto put = [&](uint16_t *hp, uint16_t *lp, int row, int col, const f32x4 &x) {
    uint2 lo;
    const uint2 hi = pack_hi(x, lo);
    const int o = row * PT + perm32(col);
    st8(hp + o, hi);
    st8(lp + o, lo);
  };
  if constexpr (STORE_T) {
    if constexpr (DELTA && RL.tcol >= 0) {
      constexpr int J = RL.tcol;
      put(&sm.th[0][0], &sm.tl[0][0], 16 * J + r, 16 * J + 4 * g, h.tdiag);
#pragma unroll
      for (int I = J + 1; I < 4; ++I) put(&sm.th[0][0], &sm.tl[0][0], 16 * I + r, 16 * J + 4 * g, h.trow[I]);
    }
    return;
  }
  int slot = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const SegWS sg = RL.seg[k];
    if (sg.kind != 2) continue;
#pragma unroll
    for (int J = 0; J <= 3; ++J)
      if (J >= sg.j0 && J <= sg.j1) put(&sm.ah[0][0], &sm.al[0][0], 16 * sg.row + r, 16 * J + 4 * g, h.a[slot][J]);
    ++slot;
  }
}


// Prep role of prep wave PW of NP (the whole loop is instantiated per wave,
// so every register it carries across the barrier has a fixed place): stages
// chunk c+1 while the state waves run chunk c. Per chunk: store the held T
// and A of chunk c and count them in (the state waves wait for that count
// only); the stagers stage the keys and queries of chunk c+1 (and issue the
// loads of chunk c+2) and count those in; then R and A, the diagonal
// inverses and the block columns of T of chunk c+1 (role_ws).
template <int PW, int NP, int GATE, bool DELTA, int D, int NSW, bool PROD, bool REV>
__device__ __forceinline__ void chunk_prep_role(const ChunkParams &p, SmemWS<D, NSW> &sm, int lane,
                                                int r, int g, int h, int hk, int64_t bos,
                                                int64_t eos, int nc) {
  using PF = PrefWS<D>;
  constexpr RoleWS RL = role_ws(DELTA, NP, PW);
  constexpr bool STAGER = RL.stager >= 0;
  // With six prep waves (delta rule) the keys are published before the
  // queries and T before A; with four, or for the linear rule, every
  // wave's part of them is published at once.
  constexpr bool SPLIT = DELTA && NP > 4;
  const int ptid = 64 * RL.stager + lane;
  PF pf;
  pf.g = pf.beta = 0.f;
  pf.gfirst = true;
  HoldWS hold;

  // Keys (KEYS) or queries of chunk ci into set ci % 2 (from pf); with the
  // keys its gate factors (first stager), with the queries the loads of
  // chunk ci + 1 into pf.
  auto stage = [&](int ci, auto keys) {
    constexpr bool KEYS = decltype(keys)::value;
    auto &S = sm.set[ci & 1];
    const int64_t t0 = bos + (int64_t)ci * C;
    const int L = (int)min<int64_t>(C, eos - t0);
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int krow = ptid / (D / 8), krs = 64 * NSTG / (D / 8), c8 = 8 * (ptid % (D / 8));
#pragma unroll
    for (int u = 0; u < PF::KU; ++u) {
      const int row = krow + u * krs;
      const bool ok = row < L;
      const uint4 x = ok ? get4(KEYS ? pf.k : pf.q, u) : z;
      uint16_t *dst = KEYS ? &S.kk[row][0] : &S.qq[row][0];
      // (8-byte aligned: rows are 16-byte multiples and perm32 keeps groups of 4)
      st8(dst + perm32(c8), make_uint2(x.x, x.y));
      st8(dst + perm32(c8 + 4), make_uint2(x.z, x.w));
    }
    if constexpr (!KEYS) {
      if (ci + 1 < nc) {
        const int64_t tn = t0 + C;
        prep_load<GATE, DELTA, D, PROD, REV>(pf, p, tn, (int)min<int64_t>(C, eos - tn), h, hk, ptid, bos + eos - 1);
      }
      return;
    }
    if constexpr (RL.stager == 0) {
      const bool ok = lane < L;
      float gl = 0.f;
      if constexpr (GATE == GDR_GATE_SCALAR) gl = ok && (!PROD || pf.gfirst) ? pf.g : 0.f;
      const float Gi = wave_scan_dpp(gl);
      const float Gl = lane_value(Gi, 63);
      S.G[lane] = Gi;
      S.eG[lane] = __expf(Gi);
      S.eGl[lane] = __expf(Gl - Gi);
      S.eB[lane] = __expf(row_bcast16<15>(Gi) - Gi);
      if (lane == 0) S.eGlast = __expf(Gl);
      S.beta[lane] = ok ? pf.beta : 0.f;
    }
  };
  using KeysT = std::true_type;
  using QueriesT = std::false_type;

  // Gram tiles, the diagonal inverse and a block column of T of chunk ci
  // (role_ws), once the stagers' key/query stores of that chunk have landed
  auto compute = [&](int ci) {
    const auto &S = sm.set[ci & 1];
    constexpr bool HAS_A = RL.seg[0].kind == 2 || RL.seg[1].kind == 2 || RL.seg[2].kind == 2 || RL.seg[3].kind == 2;
    if constexpr (DELTA && RL.seg[0].kind == 1) spin_until(&sm.kcount, NSTG * (ci + 1));
    if constexpr (DELTA) {
      gram_role<1, PW, NP, GATE, DELTA, D>(sm, S, p.scale, r, g, lane, hold);
      if constexpr (RL.inv >= 0) {
        invert_diag<RL.inv>(sm, r, g);
        count_in(&sm.rcount[RL.inv], lane);
      }
    }
    // (the queries are counted in after the keys, so this covers both)
    if constexpr (HAS_A) spin_until(&sm.qcount, NSTG * (ci + 1));
    gram_role<2, PW, NP, GATE, DELTA, D>(sm, S, p.scale, r, g, lane, hold);
    if constexpr (DELTA && RL.tcol >= 0) solve_col<RL.tcol, NP>(sm, r, g, hold, ci);
  };

  if (nc == 0) return;
  if constexpr (STAGER) {
    prep_load<GATE, DELTA, D, PROD, REV>(pf, p, bos, (int)min<int64_t>(C, eos - bos), h, hk, ptid, bos + eos - 1);
    stage(0, KeysT{});
    stage(0, QueriesT{});
    count_in(&sm.kcount, &sm.qcount, lane);
  }
  compute(0);
  __syncthreads();   // chunk 0 staged
  for (int c = 0; c < nc; ++c) {
    const bool more = c + 1 < nc;
    if constexpr (SPLIT) {
      // After the barrier (the state waves finished chunk c-1), in the order
      // the waiting waves need them, each counted in on its own: T of chunk
      // c (state waves), the keys and gate factors of chunk c+1 (R tiles),
      // its queries (A tiles), A of chunk c (state waves, later in the chunk).
      store_hold<PW, NP, DELTA, true>(sm, hold, r, g);
      count_in(&sm.tcount, lane);
      if constexpr (STAGER) {
        if (more) {
          stage(c + 1, KeysT{});
          count_in(&sm.kcount, lane);
          stage(c + 1, QueriesT{});
          count_in(&sm.qcount, lane);
        }
      }
      store_hold<PW, NP, DELTA, false>(sm, hold, r, g);
      count_in(&sm.acount, lane);
    } else {
      // T and A of chunk c, then chunk c+1 staged, two counts each
      store_hold<PW, NP, DELTA, true>(sm, hold, r, g);
      store_hold<PW, NP, DELTA, false>(sm, hold, r, g);
      count_in(&sm.tcount, &sm.acount, lane);
      if constexpr (STAGER) {
        if (more) {
          stage(c + 1, KeysT{});
          stage(c + 1, QueriesT{});
          count_in(&sm.kcount, &sm.qcount, lane);
        }
      }
    }
    if (more) compute(c + 1);
    __syncthreads();   // set c % 2, T and A are free again once the state waves are done with them
  }
}

// PROD: more than one transition per token (Gated DeltaProduct): the kernel
// runs the virtual sequence of substeps ("Linear attention visualized",
// GDP as GDN over a virtual sequence) and keeps each token's last output.
// REV: each sequence's rows walked backwards (its last row first); the
// gradients of linear attention run the forward pass this way.
// The sequence of rank `rank` when the batch is ordered longest first (ties
// by index), for batches of at most 64 sequences (lane i ranks sequence i
// against all others); larger batches keep their own order. Workgroups are
// dispatched roughly in index order and a ragged batch runs in several
// rounds of workgroups, so starting the longest sequences first shortens the
// tail. Called by whole waves.
__device__ __forceinline__ int longest_first(const int32_t *cu, int N, int rank) {
  if (N > 64) return rank;
  const int lane = threadIdx.x & 63;
  const int len = lane < N ? cu[lane + 1] - cu[lane] : -1;
  int above = 0;
  for (int i = 0; i < N; ++i) {
    const int li = scalar_load(cu + i + 1) - scalar_load(cu + i);
    above += (li > len || (li == len && i < lane)) ? 1 : 0;
  }
  const unsigned long long hit = __ballot(lane < N && above == rank);
  return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
}

// CKPT: the forward walk of the chunkwise backward; the state waves also
// store S^T at the start of every chunk to p.ckpt ([flat chunk][HV][DK][DV]
// fp32, flat chunk floor(cu[n] / 64) + n + c).
template <int GATE, bool DELTA, int D, int NSW, bool PROD, bool REV, bool CKPT = false>
__global__ __launch_bounds__(64 * (NSW + prep_waves<NSW>())) void chunk_fwd_ws_kernel(ChunkParams p) {
  constexpr int NP = prep_waves<NSW>();
  constexpr int NTH = 64 * (NSW + NP);
  using SM = SmemWS<D, NSW>;
  constexpr int BVW = 16 * NSW;
  constexpr int NB = D / BVW;
  constexpr int NT = D / 16;
  constexpr int NS = D / 32;
  constexpr int PK = SM::PK, PT = SM::PT;
  __shared__ SM sm;

  // XCD-aware decomposition (see chunk_fwd.hip); the sequences in
  // longest-first order
  const int GRP = p.ratio * NB;
  const int b = blockIdx.x;
  const int gi = (b / (8 * GRP)) * 8 + (b & 7);
  if (gi >= p.N * p.HK) return;
  const int j = (b >> 3) % GRP;
  const int rank = gi / p.HK;
  const int hk = gi - rank * p.HK;
  const int n = longest_first(p.cu_seqlens, p.N, rank);
  const int h = hk * p.ratio + j / NB;
  const int vb = j % NB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 15, g = lane >> 4;
  // the wave index through readfirstlane is provably uniform, so the role
  // branch below is a scalar branch and each role runs its own loop
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (with PROD, bos and eos count substeps: token t is rows t*P .. t*P+P-1)
  const int64_t bos = (int64_t)p.cu_seqlens[n] * (PROD ? p.P : 1);
  const int64_t eos = (int64_t)p.cu_seqlens[n + 1] * (PROD ? p.P : 1);
  const int nc = (int)((eos - bos + C - 1) / C);
  const int64_t HVD = (int64_t)p.HV * D;
  if (tid == 0)
    sm.kcount = sm.qcount = sm.tcount = sm.acount = sm.rcount[0] = sm.rcount[1] = sm.rcount[2] = sm.rcount[3] = 0;
  {
    // T and A are lower triangular: the blocks above the diagonal that their
    // fragments still read (block rows 0 and 2, next block column) stay zero
    uint4 *tz = reinterpret_cast<uint4 *>(&sm.th[0][0]);
    constexpr int NZ = 4 * C * PT * 2 / 16;   // th, tl, ah, al are contiguous
    for (int i = tid; i < NZ; i += NTH) tz[i] = make_uint4(0, 0, 0, 0);
  }
  __syncthreads();   // counters and planes initialised

  // Both roles pass the same barriers: one after the prologue and one at the
  // end of every chunk (nc + 1 in all when nc > 0, none when nc == 0).
  // Issue priority for the role that sets the pace: with six prep waves
  // (NSW = 2) the state waves' chain, with four (NSW = 4) the prep waves.
  // Each SIMD runs one wave of each kind side by side; the other fills the
  // first one's stalls. (Measured: Gated DeltaNet shapes 0.223 -> 0.216 ms
  // with the state waves first; the ragged GQA batch 1.34 -> 1.30 ms with
  // the prep waves first; the opposite choices gain nothing.)
  if (w >= NSW) {
    if constexpr (NSW == 4) __builtin_amdgcn_s_setprio(2);
#define GDR_PREP(PW) chunk_prep_role<PW, NP, GATE, DELTA, D, NSW, PROD, REV>(p, sm, lane, r, g, h, hk, bos, eos, nc)
    switch (w - NSW) {
      case 0: GDR_PREP(0); break;
      case 1: GDR_PREP(1); break;
      case 2: GDR_PREP(2); break;
      case 3: GDR_PREP(3); break;
      case 4: if constexpr (NP > 4) GDR_PREP(4); break;
      default: if constexpr (NP > 5) GDR_PREP(5); break;
    }
#undef GDR_PREP
    return;
  }

  // state waves: this lane's value column and resident state
  if constexpr (NSW == 2) __builtin_amdgcn_s_setprio(2);
  const int col = vb * BVW + 16 * w + r;
  f32x4 st[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  typename U32Vec<8>::type vreg;   // next chunk: token `lane`, this wave's 16 value columns (bf16)
  if (!p.zero_init) {
    const int64_t sbase = ((int64_t)p.slot_idx[n] * p.HV + h) * (int64_t)(D * D) + col;
    if (p.st_bf16) {
      const uint16_t *sp = static_cast<const uint16_t *>(p.pool) + sbase;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[m][i] = bf16_to_f32(sp[(16 * m + 4 * g + i) * D]);
    } else {
      const float *sp = static_cast<const float *>(p.pool) + sbase;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) st[m][i] = sp[(16 * m + 4 * g + i) * D];
    }
  }
  // The initial state loads complete here. Left in flight, they would make
  // the compiler wait inside the chunk loop for every outstanding memory
  // operation (the next chunk's value loads and this chunk's output stores)
  // before the state is first used. 0x0F70 encodes vmcnt(0) alone.
  __builtin_amdgcn_s_waitcnt(0x0F70);
  auto load_v = [&](int ci) {
    const int64_t t0 = bos + (int64_t)ci * C;
    const int last = (int)min<int64_t>(C, eos - t0) - 1;
    if constexpr (REV) {
      const int64_t bot = bos + eos - 1 - t0 - last;   // lowest memory row of the chunk
      const char *vl = static_cast<const char *>(p.v) + (bot * p.v_stride + (int64_t)h * D + vb * BVW + 16 * w) * 2;
      const uint32_t up = (uint32_t)(last - min(lane, last)) * (uint32_t)(p.v_stride * 2);
      put4(vreg, 0, *reinterpret_cast<const uint4 *>(vl + up));
      put4(vreg, 1, *reinterpret_cast<const uint4 *>(vl + up + 16));
      return;
    }
    const char *vbase = static_cast<const char *>(p.v) + (t0 * p.v_stride + (int64_t)h * D + vb * BVW + 16 * w) * 2;
    const uint32_t off = (uint32_t)min(lane, last) * (uint32_t)(p.v_stride * 2);
    put4(vreg, 0, *reinterpret_cast<const uint4 *>(vbase + off));
    put4(vreg, 1, *reinterpret_cast<const uint4 *>(vbase + off + 16));
  };
  // A zero-length sequence has no rows to read and its prep waves have
  // already left, so it goes straight to the write-back of its initial state.
  if (nc > 0) {
    load_v(0);
    __syncthreads();   // chunk 0 staged by the prep waves
  }

  for (int c = 0; c < nc; ++c) {
    if constexpr (CKPT) {
      const int64_t F = (int64_t)(p.cu_seqlens[n] >> 6) + n + c;
      float *cp = p.ckpt + (F * p.HV + h) * (int64_t)(D * D) + col;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) cp[(16 * m + 4 * g + i) * D] = st[m][i];
    }
    {
      const auto &S = sm.set[c & 1];
      const int64_t t0 = bos + (int64_t)c * C;
      const int L = (int)min<int64_t>(C, eos - t0);

      // This chunk's values go to this wave's LDS tile (16-byte halves
      // swapped on rows with bit 3 set, so the row writes do not collide) and
      // come back in the accumulator layout through transposing reads; the
      // next chunk's loads go in flight.
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      uint16_t *vx = &sm.vx[w][0][0];
      {
        const uint4 z = make_uint4(0, 0, 0, 0);
        const bool okv = lane < L;
        const int sw = (lane >> 3) & 1;
        st16(vx + lane * 16 + 8 * sw, okv ? get4(vreg, 0) : z);
        st16(vx + lane * 16 + 8 * (sw ^ 1), okv ? get4(vreg, 1) : z);
        if (c + 1 < nc) load_v(c + 1);
      }

      // The state split once per key step (B operand of X and of Q S^T), and
      // X = K S^T (delta rule): the split and the key fragments of step s+1
      // are formed while step s multiplies.
      Frag sf[NS];
      f32x4 xa[4], qa[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) xa[I] = qa[I] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (DELTA) {
        Frag fk[2][4];
#pragma unroll
        for (int I = 0; I < 4; ++I) ldfrag(&S.kk[0][0], PK, 16 * I + r, 0, g, fk[0][I]);
        chainfrag(st[0], st[1], sf[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s + 1 < NS) {
#pragma unroll
            for (int I = 0; I < 4; ++I) ldfrag(&S.kk[0][0], PK, 16 * I + r, 32 * (s + 1), g, fk[(s + 1) & 1][I]);
          }
#pragma unroll
          for (int I = 0; I < 4; ++I) xa[I] = mm_pass<1, false, true>(fk[s & 1][I], sf[s], xa[I]);
#pragma unroll
          for (int I = 0; I < 4; ++I) xa[I] = mm_pass<2, false, true>(fk[s & 1][I], sf[s], xa[I]);
          if (s + 1 < NS) chainfrag(st[2 * s + 2], st[2 * s + 3], sf[s + 1]);
          interleave<8, 3, 1>();
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int s = 0; s < NS; ++s) chainfrag(st[2 * s], st[2 * s + 1], sf[s]);
      }

      // Q S^T. Its first query fragments and the values' transposing reads
      // issue before the wait for T and A of this chunk (in LDS once every
      // prep wave has stored them); T's fragments load, and the values and
      // (delta rule) the split right-hand side beta (V - e^{G} X) of the
      // solve are formed, under its products.
      Frag fq[2][4];
#pragma unroll
      for (int I = 0; I < 4; ++I) ldfrag(&S.qq[0][0], PK, 16 * I + r, 0, g, fq[0][I]);
      s16x4 vtr[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int row = 16 * I + 4 * g + (r >> 2);
        const int half = ((r & 3) >> 1) ^ ((row >> 3) & 1);
        vtr[I] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(vx + row * 16 + 8 * half + 4 * (r & 1)));
      }
      spin_until(&sm.tcount, NP * (c + 1));
      Frag tf[4][2];
      float4 Bi[4], Ei[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        Ei[I] = ld4(&S.eG[16 * I + 4 * g]);
        if constexpr (DELTA) {
          Bi[I] = ld4(&S.beta[16 * I + 4 * g]);
#pragma unroll
          for (int s = 0; s <= (I >> 1); ++s) ldfrag2(&sm.th[0][0], &sm.tl[0][0], PT, 16 * I + r, s, g, tf[I][s]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x4 vt[4], rv[4];
      Frag rb[2];
      // vector work under step s: the values (item 0), beta (V - e^{G} X)
      // for blocks 0-1 and 2-3 (items 1, 2), its two splits (items 3, 4)
      auto item = [&](int k) {
        if (k == 0) {
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) vt[I][i] = bf16_to_f32((uint16_t)vtr[I][i]);
        } else if (k <= 2) {
#pragma unroll
          for (int I = 2 * k - 2; I < 2 * k; ++I) {
            const float bi[4] = {Bi[I].x, Bi[I].y, Bi[I].z, Bi[I].w};
            const float ei[4] = {Ei[I].x, Ei[I].y, Ei[I].z, Ei[I].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = xa[I][i];
              if constexpr (GATE == GDR_GATE_SCALAR) x *= ei[i];
              rv[I][i] = bi[i] * (vt[I][i] - x);
            }
          }
        } else {
          chainfrag(rv[2 * k - 6], rv[2 * k - 5], rb[k - 3]);
        }
      };
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s + 1 < NS) {
#pragma unroll
          for (int I = 0; I < 4; ++I) ldfrag(&S.qq[0][0], PK, 16 * I + r, 32 * (s + 1), g, fq[(s + 1) & 1][I]);
        }
#pragma unroll
        for (int I = 0; I < 4; ++I) qa[I] = mm_pass<1, false, true>(fq[s & 1][I], sf[s], qa[I]);
#pragma unroll
        for (int I = 0; I < 4; ++I) qa[I] = mm_pass<2, false, true>(fq[s & 1][I], sf[s], qa[I]);
        // items by step: 0 | 1 | 2 3 | 4 over four steps, 0 1 2 | 3 4 over two
#pragma unroll
        for (int k = 0; k < (DELTA ? 5 : 1); ++k) {
          const int at = NS == 4 ? (k < 2 ? k : k < 4 ? 2 : 3) : (k < 3 ? 0 : 1);
          if (at == s) item(k);
        }
        interleave<8, 6, 1>();
        __builtin_amdgcn_sched_barrier(0);
      }

      // Vb = T (beta (V - e^{G} X)) (delta rule) or V (linear rule): blocks
      // 0-1 first, whose split for O is formed while blocks 2-3 multiply;
      // A's fragments load and the query part of O and the state decay are
      // scaled meanwhile
      f32x4 vbar[4];
      Frag af[4][2], vbf[2];
      spin_until(&sm.acount, NP * (c + 1));
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int s = 0; s <= (I >> 1); ++s) ldfrag2(&sm.ah[0][0], &sm.al[0][0], PT, 16 * I + r, s, g, af[I][s]);
      if constexpr (DELTA) {
#pragma unroll
        for (int I = 0; I < 4; ++I) vbar[I] = f32x4{0.f, 0.f, 0.f, 0.f};
        // (k step 0 for all four blocks, then step 1 for blocks 2-3)
        auto vpass = [&](auto P, int s) {
#pragma unroll
          for (int I = 2 * s; I < 4; ++I)
            vbar[I] = mm_pass<decltype(P)::value, true, true>(tf[I][s], rb[s], vbar[I]);
        };
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          vpass(std::integral_constant<int, 0>{}, s);
          vpass(std::integral_constant<int, 1>{}, s);
          vpass(std::integral_constant<int, 2>{}, s);
        }
      } else {
#pragma unroll
        for (int I = 0; I < 4; ++I) vbar[I] = vt[I];
      }
      chainfrag(vbar[0], vbar[1], vbf[0]);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const float ei[4] = {Ei[I].x, Ei[I].y, Ei[I].z, Ei[I].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sc = p.scale;
          if constexpr (GATE == GDR_GATE_SCALAR) sc *= ei[i];
          qa[I][i] *= sc;
        }
      }
      if constexpr (GATE == GDR_GATE_SCALAR) {
        const float a = S.eGlast;
#pragma unroll
        for (int m = 0; m < NT; ++m) st[m] *= a;
      }
      if constexpr (DELTA) interleave<18, 5, 0>();
      __builtin_amdgcn_sched_barrier(0);

      // O = s e^{G} (.) Q S^T + A Vb: the products with Vb blocks 0-1 first,
      // while the split of blocks 2-3, the values of the state update
      // e^{G_last - G} Vb (split) and its key fragments (transposing reads)
      // are formed and loaded.
      Frag kt[NT][2];
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int s = 0; s < 2; ++s) ldfrag_kt(&S.kk[0][0], PK, m, s, r, g, kt[m][s]);
      f32x4 oa[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) oa[I] = mm_pass<0, true, DELTA>(af[I][0], vbf[0], qa[I]);
#pragma unroll
      for (int I = 0; I < 4; ++I) oa[I] = mm_pass<1, true, DELTA>(af[I][0], vbf[0], oa[I]);
#pragma unroll
      for (int I = 0; I < 4; ++I) oa[I] = mm_pass<2, true, DELTA>(af[I][0], vbf[0], oa[I]);
      chainfrag(vbar[2], vbar[3], vbf[1]);
      Frag uf[2];
      {
        f32x4 vs[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const float4 El = ld4(&S.eGl[16 * I + 4 * g]);
          const float el[4] = {El.x, El.y, El.z, El.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = vbar[I][i];
            if constexpr (GATE == GDR_GATE_SCALAR) x *= el[i];
            vs[I][i] = x;
          }
        }
        chainfrag(vs[0], vs[1], uf[0]);
        chainfrag(vs[2], vs[3], uf[1]);
      }
#pragma unroll
      for (int I = 2; I < 4; ++I) oa[I] = mm_pass<0, true, DELTA>(af[I][1], vbf[1], oa[I]);
#pragma unroll
      for (int I = 2; I < 4; ++I) oa[I] = mm_pass<1, true, DELTA>(af[I][1], vbf[1], oa[I]);
#pragma unroll
      for (int I = 2; I < 4; ++I) oa[I] = mm_pass<2, true, DELTA>(af[I][1], vbf[1], oa[I]);
      interleave<DELTA ? 18 : 12, 6, 0>();
      __builtin_amdgcn_sched_barrier(0);

      // S^T <- e^{G_last} S^T + K^T (e^{G_last - G_j} Vb_j), then this
      // chunk's outputs
      {
        constexpr bool USPLIT = DELTA || GATE == GDR_GATE_SCALAR;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
          for (int m = 0; m < NT; ++m) st[m] = mm_pass<1, false, USPLIT>(kt[m][s], uf[s], st[m]);
#pragma unroll
          for (int m = 0; m < NT; ++m) st[m] = mm_pass<2, false, USPLIT>(kt[m][s], uf[s], st[m]);
        }
      }
      {
        // Buffer stores against a descriptor over this chunk's 64 output
        // rows: row 16I + i is a scalar offset, the lane part (row group 4g,
        // column) a fixed 32-bit offset, so no per-store address arithmetic.
        const uint32_t HVDu = (uint32_t)HVD;
        const uint32_t osz = p.out_bf16 ? 2u : 4u;
        char *obase = static_cast<char *>(p.o) + (t0 * HVD + (int64_t)h * D) * osz;
        const uint32_t orow = HVDu * osz;
        const __amdgpu_buffer_rsrc_t ors =
            __builtin_amdgcn_make_buffer_rsrc(obase, 0, (int)(C * orow), 0x00020000);
        const uint32_t olane = ((uint32_t)(4 * g) * HVDu + (uint32_t)col) * osz;
        // (uniform branches: a full chunk stores unmasked; rows past a
        // partial chunk's end are skipped)
        if constexpr (REV) {
          // Row t0 + ii of the walk is memory row bos + eos - 1 - (t0 + ii).
          // The descriptor starts at the lowest of the chunk's L rows and
          // spans L rows, so row ii sits (L - 1 - ii) rows up; rows past
          // the chunk's end (ii >= L) wrap to huge offsets and are dropped
          // by the descriptor's range check.
          char *rbase = static_cast<char *>(p.o) + ((bos + eos - 1 - t0 - (L - 1)) * HVD + (int64_t)h * D) * osz;
          const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(rbase, 0, (int)(L * orow), 0x00020000);
          const uint32_t rlane = (uint32_t)(L - 1 - 4 * g) * orow + (uint32_t)col * osz;
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t voff = rlane - (uint32_t)(16 * I + i) * orow;
              if (p.out_bf16)
                __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(oa[I][i]), rrs, voff, 0, 0);
              else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oa[I][i]), rrs, voff, 0, 0);
            }
        } else if constexpr (PROD) {
          // a token's output is its last substep's: row t0 + ii goes to o
          // row (t0 + ii) / P when it is one, and is dropped otherwise
          const SubMap map(t0, p.P);
          char *ocol = static_cast<char *>(p.o) + ((map.r0 * HVD + (int64_t)h * D + col) * osz);
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ii = 16 * I + 4 * g + i;
              if (ii < L && map.sub(ii) == map.P - 1) {
                char *dst = ocol + (int64_t)map.tok(ii) * HVD * osz;
                if (p.out_bf16) *reinterpret_cast<uint16_t *>(dst) = f32_to_bf16(oa[I][i]);
                else *reinterpret_cast<float *>(dst) = oa[I][i];
              }
            }
        } else if (!p.out_bf16) {
          if (L == C) {
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oa[I][i]), ors, olane,
                                                      (16 * I + i) * (int)orow, 0);
          } else {
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (16 * I + 4 * g + i < L)
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oa[I][i]), ors, olane,
                                                        (16 * I + i) * (int)orow, 0);
          }
        } else {
          // (pairs converted by one packed instruction; the high half stored
          // from the same register)
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              const bf16x2 pr = {static_cast<__bf16>(oa[I][i]), static_cast<__bf16>(oa[I][i + 1])};
              const uint32_t u = __builtin_bit_cast(uint32_t, pr);
              if (L == C || 16 * I + 4 * g + i < L)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)u, ors, olane, (16 * I + i) * (int)orow, 0);
              if (L == C || 16 * I + 4 * g + i + 1 < L)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(u >> 16), ors, olane,
                                                      (16 * I + i + 1) * (int)orow, 0);
            }
        }
      }
    }
    __syncthreads();   // set c % 2, T and A are refilled by the prep waves next
  }

  // ---- final state back to the pool slot ----
  {
    const int64_t sbase = ((int64_t)p.slot_idx[n] * p.HV + h) * (int64_t)(D * D) + col;
    if (p.st_bf16) {
      uint16_t *sp = static_cast<uint16_t *>(p.pool) + sbase;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[(16 * m + 4 * g + i) * D] = f32_to_bf16(st[m][i]);
    } else {
      float *sp = static_cast<float *>(p.pool) + sbase;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) sp[(16 * m + 4 * g + i) * D] = st[m][i];
    }
  }
}


template <int GATE, bool DELTA, int D, int NSW>
hipError_t launch_ws(const ChunkParams &p, hipStream_t stream) {
  const int grp = p.ratio * (D / (16 * NSW));
  const int blocks = ((p.N * p.HK + 7) / 8) * 8 * grp;
  if (p.P > 1)
    hipLaunchKernelGGL((chunk_fwd_ws_kernel<GATE, DELTA, D, NSW, true, false>), dim3(blocks),
                       dim3(64 * (NSW + prep_waves<NSW>())), 0, stream, p);
  else if (p.rev) {
    // (the reversed walk serves the linear-attention gradients only, plain
    // or with a scalar gate)
    if constexpr (!DELTA)
      hipLaunchKernelGGL((chunk_fwd_ws_kernel<GATE, DELTA, D, NSW, false, true>), dim3(blocks),
                         dim3(64 * (NSW + prep_waves<NSW>())), 0, stream, p);
    else
      return hipErrorInvalidValue;
  } else
    hipLaunchKernelGGL((chunk_fwd_ws_kernel<GATE, DELTA, D, NSW, false, false>), dim3(blocks),
                       dim3(64 * (NSW + prep_waves<NSW>())), 0, stream, p);
  return hipGetLastError();
}

template <int GATE, int D>
hipError_t launch_ws_ckpt(const ChunkParams &p, hipStream_t stream) {
  const int64_t wide = (int64_t)p.N * p.HV * (D / 64);
  auto go = [&](auto nsw) {
    constexpr int NSW = decltype(nsw)::value;
    const int grp = p.ratio * (D / (16 * NSW));
    const int blocks = ((p.N * p.HK + 7) / 8) * 8 * grp;
    hipLaunchKernelGGL((chunk_fwd_ws_kernel<GATE, true, D, NSW, false, false, true>), dim3(blocks),
                       dim3(64 * (NSW + prep_waves<NSW>())), 0, stream, p);
    return hipGetLastError();
  };
  if (wide >= cu_count()) return go(std::integral_constant<int, 4>());
  return go(std::integral_constant<int, 2>());
}

// 64 value columns per workgroup when that already gives every compute unit
// a workgroup, else 32 (twice the workgroups, each with half the state work).
template <int GATE, bool DELTA, int D>
hipError_t ws_by_width(const ChunkParams &p, hipStream_t s) {
  const int64_t wide = (int64_t)p.N * p.HV * (D / 64);
  if (wide >= cu_count()) return launch_ws<GATE, DELTA, D, 4>(p, s);
  return launch_ws<GATE, DELTA, D, 2>(p, s);
}

template <int GATE, bool DELTA>
hipError_t ws_by_dim(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.DK == 128) return ws_by_width<GATE, DELTA, 128>(p, s);
  return ws_by_width<GATE, DELTA, 64>(p, s);
}

template <int GATE>
hipError_t ws_by_rule(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.rule == GDR_RULE_DELTA) return ws_by_dim<GATE, true>(a, p, s);
  return ws_by_dim<GATE, false>(a, p, s);
}

}  // namespace

// Compute units of the current device (cached per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t ws_wait_flag(int *out, bool clear, hipStream_t stream) {
  return chunk::wait_flag_access(out, clear, stream);
}

// The backward's forward walk on this kernel (bf16 inputs, delta rule, gate
// NONE or SCALAR): outputs to a.o and the final state to a.state_pool as
// usual (the caller passes scratch for both), and S^T at every chunk start
// to ckpt.
hipError_t launch_chunk_states_ws(const gdr_args &a, float *ckpt, hipStream_t stream) {
  ChunkParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = a.o; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HK = a.HK; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  p.P = 1;
  p.rev = 0;
  p.lc = 64;
  p.ckpt = ckpt;
  if (a.gate == GDR_GATE_SCALAR)
    return a.DK == 128 ? launch_ws_ckpt<GDR_GATE_SCALAR, 128>(p, stream) : launch_ws_ckpt<GDR_GATE_SCALAR, 64>(p, stream);
  return a.DK == 128 ? launch_ws_ckpt<GDR_GATE_NONE, 128>(p, stream) : launch_ws_ckpt<GDR_GATE_NONE, 64>(p, stream);
}

hipError_t launch_chunk_fwd_ws(const gdr_args &a, hipStream_t stream) {
  ChunkParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = a.o; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HK = a.HK; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = a.out_dtype == GDR_BF16;
  p.P = products_of(a);
  p.rev = (a.flags & kFlagReverse) ? 1 : 0;
  p.lc = 64;
  p.ckpt = nullptr;
  if (a.gate == GDR_GATE_SCALAR) return ws_by_rule<GDR_GATE_SCALAR>(a, p, stream);
  return ws_by_rule<GDR_GATE_NONE>(a, p, stream);
}

}  // namespace gdr
