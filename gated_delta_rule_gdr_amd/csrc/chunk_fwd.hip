// Chunkwise prefill of the gated delta rule on gfx950 MFMA.
//
// Math (one value head, chunk of C = 64 tokens, incoming state S, value-by-key;
// section 6 of "You Could Have Come Up With Kimi Delta Attention" and section
// 4 of "From Attention to Learned Memory"). With the inclusive in-chunk
// cumulative log-decay G_i (per key channel for the channel gate):
//   R   = strict-lower( beta_i k_i^T D_{j+1:i} k_j )       key-key coefficients
//   A   = lower( s q_i^T D_{j+1:i} k_j )                    query-key coefficients
//   X   = (D_{0:i} k_i)^T S^T  rows                         prediction of the incoming state
//   Vb  = (I + R)^-1 (beta (V - X))                         solved errors e_i
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
// matrices on MFMA; the inverses T_II of the four 16x16 diagonal blocks of
// I + R by forward substitution (section 4 of "From Attention to Learned
// Memory" builds the 64x64 inverse from these blocks); then each wave's
// state-dependent products on MFMA, where the 64-row unit lower triangular
// system is solved blockwise on the right-hand side itself,
// Vb_I = T_II (R_v,I - sum_{J<I} R_IJ Vb_J), so the full inverse is never
// formed.
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
// the key contraction. The Gram entries are summed pair by pair over the
// channels with the factor e^{G_i - G_j} (j <= i) of each channel, the
// token-parallel form of the diagonal interaction blocks on the KDA page
// (section 6); the state products use e^{G} (.) q, e^{G} (.) k and the keys
// decayed to the chunk's end, e^{G_last - G} (.) k. Every exponent is <= 0,
// so no gate, however strong, can overflow a factor.
//
// MFMA fragment convention (v_mfma_f32_16x16x32_bf16, wave64, lane l,
// r = l % 16, g = l / 16): an A fragment holds A[r][k] and a B fragment
// B[k][r] for the eight k of slot set K(g) = {4g..4g+3} u {16+4g..16+4g+3}
// of a 32-wide k step; the product pairs equal slots of A and B, so any fixed
// k labelling works as long as A and B agree. The accumulator holds
// C[4g + i][r], i = 0..3. With K(g) so chosen, two stacked 16-row accumulator
// tiles are directly the B fragment of the next product that contracts over
// those rows: no data movement between chained products.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "chunk_common.h"

namespace gdr {
namespace {

using namespace chunk;

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
  static constexpr int PB = C + 8;                 // bf16 C x C planes
  Op kk[C][PK];   // keys (channel: e^{G} k) - A operand of X, rows of R
  Op qq[C][PK];   // queries (channel: e^{G} q; first the raw queries)
  // Transposed keys for the state update (channel: the keys decayed to the
  // chunk's end, e^{G_last - G} k). For the channel gate the same storage
  // first holds the raw keys token-major for the Gram entries.
  union {
    Op kt[D][PT];
    Op kinv[C][PK];
  };
  In vv[C][PV];   // this workgroup's value columns
  // The C x C coefficient matrices, already split into bf16 hi / lo planes:
  // R's off-diagonal blocks and the diagonal-block inverses T_II share rt*,
  // A sits in aq*. rd holds R's diagonal blocks in fp32 for the solve. During the channel-gate prep the same storage stages g.
  union {
    struct {
      uint16_t rth[C][PB], rtl[C][PB];
      uint16_t aqh[C][PB], aql[C][PB];
      float rd[4][16][20];
    };
    float gstage[C][D];
  };
  float G[C], eG[C], eGl[C], beta[C];
  float eGlastc[D];
  float eGlast;
};

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

// Registers holding one chunk's keys, queries, values and gates between its
// global loads and its LDS stores, so that the loads of chunk c+1 are in
// flight while chunk c computes.
template <bool IN_F32, int D>
struct Prefetch {
  static constexpr int E = IN_F32 ? 4 : 8;       // elements per 16-byte unit
  static constexpr int KU = C * D / E / 256;     // units per thread, keys (and queries)
  static constexpr int VU = C * BV / E / 256;    // units per thread, values
  typename U32Vec<4 * KU>::type k, q;
  typename U32Vec<4 * VU>::type v;
  float g, beta;                                 // wave 0: token `lane`
  bool gfirst;                                   // wave 0: row `lane` is a token's first substep
};

// Where each lane's prefetch units sit inside a chunk: unit u of the keys is
// row krow + u * krs, 16-byte column block kc (same for queries); values
// likewise with vrow / vrs / vc.
struct LaneOffsets {
  int krow, krs, kc;
  int vrow, vrs, vc;
};

template <bool IN_F32, int D>
__device__ __forceinline__ LaneOffsets lane_offsets() {
  using PF = Prefetch<IN_F32, D>;
  constexpr int E = PF::E;
  const int tid = threadIdx.x;
  LaneOffsets o;
  o.krow = tid / (D / E);
  o.krs = 256 / (D / E);
  o.kc = (tid % (D / E)) * 16;
  o.vrow = tid / (BV / E);
  o.vrs = 256 / (BV / E);
  o.vc = (tid % (BV / E)) * 16;
  return o;
}

// Issue the global loads of the chunk starting at token t0 (L valid rows).
// Rows past the chunk's end are clamped to its last row so every load is in
// bounds and unconditional; they are zeroed when stored to LDS. No load is
// waited for here: the registers are consumed by the next chunk's LDS stores.
template <bool IN_F32, int GATE, bool DELTA, int D>
__device__ __forceinline__ void load_chunk(Prefetch<IN_F32, D> &pf, const ChunkParams &p,
                                           const LaneOffsets &lo, int64_t t0, int L, int h,
                                           int hk, int vb) {
  using PF = Prefetch<IN_F32, D>;
  constexpr int es = IN_F32 ? 4 : 2;
  // rows are substeps when P > 1: keys, values and beta by substep, the
  // query and gate of the substep's token (the gate on its first substep)
  const SubMap map(t0, p.P);
  const char *kb = static_cast<const char *>(p.k) + (t0 * p.k_stride + (int64_t)hk * D) * es;
  const char *qb = static_cast<const char *>(p.q) + (map.r0 * p.q_stride + (int64_t)hk * D) * es;
  const char *vb_ = static_cast<const char *>(p.v) + (t0 * p.v_stride + (int64_t)h * D + vb * BV) * es;
  const uint32_t ks = (uint32_t)(p.k_stride * es), qs = (uint32_t)(p.q_stride * es),
                 vs = (uint32_t)(p.v_stride * es);
  const int last = L - 1;
#pragma unroll
  for (int u = 0; u < PF::KU; ++u) {
    const uint32_t row = (uint32_t)min(lo.krow + u * lo.krs, last);
    const uint32_t qr = (uint32_t)map.tok((int)row);
    put4(pf.k, u, *reinterpret_cast<const uint4 *>(kb + (row * ks + lo.kc)));
    put4(pf.q, u, *reinterpret_cast<const uint4 *>(qb + (qr * qs + lo.kc)));
  }
#pragma unroll
  for (int u = 0; u < PF::VU; ++u) {
    const uint32_t row = (uint32_t)min(lo.vrow + u * lo.vrs, last);
    put4(pf.v, u, *reinterpret_cast<const uint4 *>(vb_ + (row * vs + lo.vc)));
  }
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int row = min(tid, last);
    if constexpr (GATE == GDR_GATE_SCALAR) pf.g = p.g[(map.r0 + map.tok(row)) * p.HV + h];
    pf.gfirst = map.sub(row) == 0;
    if constexpr (DELTA) pf.beta = p.beta[(t0 + row) * p.HV + h];
  }
}

// Gram matrices of one chunk, lower 16x16 tiles (I >= J). Delta rule: waves
// 0-1 form K K^T (-> R), waves 2-3 form Q K^T (-> A); each wave owns row
// blocks {a, 3-a} (five tiles, their fragments loaded once, five independent
// MFMA chains). Linear rule: wave w forms the Q K^T tiles of row block w. The
// wave's role is a template argument so each role is straight-line code.
// Each tile is computed transposed (keys of block J as the M operand, rows of
// block I as N), so a lane ends up holding row ii = 16I + r, columns
// jj = 16J + 4g .. +3: exactly the A-fragment layout of the 16x16x16 products
// that consume R and A, stored with one 8-byte write per plane.
template <int W, bool IN_F32, int GATE, bool DELTA, int D, class SM>
__device__ __forceinline__ void grams(SM &sm, const ChunkParams &p, int r, int g) {
  constexpr bool OPF32 = SM::OPF32;
  constexpr int NS = D / 32;
  constexpr bool ISQ = DELTA ? (W >= 2) : true;
  constexpr int IA = DELTA ? (W & 1) : W;
  constexpr int NRB = DELTA ? 2 : 1;
  constexpr int IB = DELTA ? 3 - IA : IA;
  constexpr int JMAX = IB > IA ? IB : IA;
  using Op = typename SM::Op;
  const Op *nrow = ISQ ? &sm.qq[0][0] : &sm.kk[0][0];

  Frag fn[NRB][NS];   // rows of blocks IA, IB (N operand)
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ldfrag(nrow, SM::PK, 16 * IA + r, 32 * s, g, fn[0][s]);
    if constexpr (DELTA) ldfrag(nrow, SM::PK, 16 * IB + r, 32 * s, g, fn[NRB - 1][s]);
  }
  f32x4 acc[NRB][4];
#pragma unroll
  for (int J = 0; J <= JMAX; ++J) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[rb][J] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag fm[NS];   // keys of block J (M operand)
#pragma unroll
    for (int s = 0; s < NS; ++s) ldfrag(&sm.kk[0][0], SM::PK, 16 * J + r, 32 * s, g, fm[s]);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int I = rb ? IB : IA;
      if (J <= I) {
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[rb][J] = mm<OPF32, OPF32>(fm[s], fn[rb][s], acc[rb][J]);
      }
    }
  }
  // decay, write strength, mask; store split planes (+ R's diagonal in fp32)
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int I = rb ? IB : IA;
    const int ii = 16 * I + r;
    const float Gi = sm.G[ii], bi = sm.beta[ii];
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      const float4 Gj4 = *reinterpret_cast<const float4 *>(&sm.G[16 * J + 4 * g]);
      const float Gj[4] = {Gj4.x, Gj4.y, Gj4.z, Gj4.w};
      float val[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = 16 * J + 4 * g + i;
        float gam = 1.f;
        if constexpr (GATE == GDR_GATE_SCALAR) gam = __expf(Gi - Gj[i]);
        if constexpr (ISQ) val[i] = (jj <= ii) ? p.scale * acc[rb][J][i] * gam : 0.f;
        else val[i] = (jj < ii) ? bi * acc[rb][J][i] * gam : 0.f;
      }
      if (!ISQ && J == I) {
        *reinterpret_cast<float4 *>(&sm.rd[I][r][4 * g]) = make_float4(val[0], val[1], val[2], val[3]);
      } else {
        uint16_t hb[4], lb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 hh = static_cast<__bf16>(val[i]);
          hb[i] = __builtin_bit_cast(uint16_t, hh);
          lb[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(val[i] - static_cast<float>(hh)));
        }
        const uint2 hw = make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
        const uint2 lw = make_uint2(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16));
        uint16_t *ph = ISQ ? &sm.aqh[0][0] : &sm.rth[0][0];
        uint16_t *pl = ISQ ? &sm.aql[0][0] : &sm.rtl[0][0];
        *reinterpret_cast<uint2 *>(ph + ii * SM::PB + 16 * J + 4 * g) = hw;
        *reinterpret_cast<uint2 *>(pl + ii * SM::PB + 16 * J + 4 * g) = lw;
      }
    }
  }
}

// CKPT: the forward walk of the chunkwise backward. The state at the start
// of every chunk goes to p.ckpt (fp32 S^T, [flat chunk][HV][DK][DV], flat
// chunk base(n) + c with base(n) = floor(cu[n] / 64) + n), and neither the
// outputs nor the final state are written.
template <bool IN_F32, int GATE, bool DELTA, int D, bool CKPT = false>
__global__ __launch_bounds__(256) void chunk_fwd_kernel(ChunkParams p) {
  using SM = Smem<IN_F32, GATE, DELTA, D>;
  using In = typename SM::In;
  using PF = Prefetch<IN_F32, D>;
  constexpr bool OPF32 = SM::OPF32;
  constexpr int NB = D / BV;
  constexpr int NT = D / 16;   // 16-row tiles over the key dim
  constexpr int NS = D / 32;   // 32-wide k steps over the key dim
  __shared__ SM sm;

  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2). All workgroups that read the same keys and queries - the value
  // blocks of the value heads sharing one key head of one sequence - get ids
  // that are equal modulo 8, so they run on one XCD and share those reads.
  const int GRP = p.ratio * NB;                 // workgroups per (sequence, key head)
  const int b = blockIdx.x;
  const int gi = (b / (8 * GRP)) * 8 + (b & 7);  // (sequence, key head) group
  if (gi >= p.N * p.HK) return;                 // padding of the last XCD round
  const int j = (b >> 3) % GRP;
  const int n = gi / p.HK;
  const int hk = gi - n * p.HK;
  const int h = hk * p.ratio + j / NB;
  const int vb = j % NB;
  const int tid = threadIdx.x;
  // (the wave index through readfirstlane: the compiler then knows it is
  // uniform, so the role switches below are scalar branches, never
  // exec-masked regions around MFMAs)
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, r = lane & 15, g = lane >> 4;
  const int col = vb * BV + 16 * w + r;   // value column this lane owns in C tiles

  // bos and eos count substeps: token t is rows t*P .. t*P+P-1 (P = 1 but
  // for Gated DeltaProduct, run as GDN over its virtual sequence)
  const int64_t bos = (int64_t)p.cu_seqlens[n] * p.P, eos = (int64_t)p.cu_seqlens[n + 1] * p.P;
  const int64_t slot = p.slot_idx[n];

  // ---- initial state: st[m][i] = S^T[16m + 4g + i][col] ----
  f32x4 st[NT];
  {
    const int64_t sbase = (slot * p.HV + h) * (int64_t)(D * D) + col;
#pragma unroll
    for (int m = 0; m < NT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (!p.zero_init) {
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
  }

  // The initial state loads complete here, so that the chunk loop never
  // waits on them (and hence on everything issued after them). 0x0F70
  // encodes vmcnt(0) alone.
  __builtin_amdgcn_s_waitcnt(0x0F70);

  PF pf;
  pf.g = pf.beta = 0.f;
  pf.gfirst = true;
  const LaneOffsets lo = lane_offsets<IN_F32, D>();
  if constexpr (GATE != GDR_GATE_CHANNEL) {
    if (bos < eos)
      load_chunk<IN_F32, GATE, DELTA, D>(pf, p, lo, bos, (int)min<int64_t>(p.lc, eos - bos), h, hk, vb);
  }

  // Chunks of LC = 16, 32 or 64 tokens: a shorter chunk runs in the 64-row
  // tile with its rows past LC zero, the same path as a sequence's last,
  // partial chunk (the state is carried every LC tokens, which is the
  // chunked algorithm at that chunk length).
  const int LC = p.lc;
  const int64_t HVD = (int64_t)p.HV * D;
  for (int64_t t0 = bos; t0 < eos; t0 += LC) {
    const int L = (int)((eos - t0) < LC ? (eos - t0) : LC);
    if constexpr (CKPT) {
      const int64_t F = (int64_t)(p.cu_seqlens[n] >> 6) + n + (t0 - bos) / C;
      float *cp = p.ckpt + (F * p.HV + h) * (int64_t)(D * D) + col;
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) cp[(16 * m + 4 * g + i) * D] = st[m][i];
    }

    // ================= phase 0: inputs into LDS =================
    if constexpr (GATE != GDR_GATE_CHANNEL) {
      const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < PF::KU; ++u) {
        const int row = lo.krow + u * lo.krs, c = lo.kc / (int)sizeof(In);
        const bool ok = row < L;
        const uint4 kx = ok ? get4(pf.k, u) : z, qx = ok ? get4(pf.q, u) : z;
        if constexpr (IN_F32) {   // 4 columns: one permuted group
          *reinterpret_cast<uint4 *>(&sm.kk[row][perm32(c)]) = kx;
          *reinterpret_cast<uint4 *>(&sm.qq[row][perm32(c)]) = qx;
        } else {                  // 8 columns: two permuted groups of 4
          *reinterpret_cast<uint2 *>(&sm.kk[row][perm32(c)]) = make_uint2(kx.x, kx.y);
          *reinterpret_cast<uint2 *>(&sm.kk[row][perm32(c + 4)]) = make_uint2(kx.z, kx.w);
          *reinterpret_cast<uint2 *>(&sm.qq[row][perm32(c)]) = make_uint2(qx.x, qx.y);
          *reinterpret_cast<uint2 *>(&sm.qq[row][perm32(c + 4)]) = make_uint2(qx.z, qx.w);
        }
      }
#pragma unroll
      for (int u = 0; u < PF::VU; ++u) {
        const int row = lo.vrow + u * lo.vrs, c = lo.vc / (int)sizeof(In);
        *reinterpret_cast<uint4 *>(&sm.vv[row][c]) = row < L ? get4(pf.v, u) : z;
      }
      if (w == 0) {
        const bool ok = lane < L;
        float gl = 0.f;
        if constexpr (GATE == GDR_GATE_SCALAR) gl = ok && pf.gfirst ? pf.g : 0.f;
        const float Gi = wave_scan(gl);
        const float Gl = __shfl(Gi, 63, 64);
        sm.G[lane] = Gi;
        sm.eG[lane] = __expf(Gi);
        sm.eGl[lane] = __expf(Gl - Gi);
        if (lane == 0) sm.eGlast = __expf(Gl);
        sm.beta[lane] = ok ? pf.beta : 0.f;
      }
      // next chunk's loads stay in flight while this one computes
      if (t0 + LC < eos)
        load_chunk<IN_F32, GATE, DELTA, D>(pf, p, lo, t0 + LC, (int)min<int64_t>(LC, eos - t0 - LC), h,
                                           hk, vb);
      __syncthreads();
      // transposed keys for the state update (read only at the end of the chunk)
      constexpr int E = PF::E;
      constexpr int RG = C / E;   // row groups of E tokens
#pragma unroll
      for (int u = 0; u < D * RG / 256; ++u) {
        const int it = tid + 256 * u, dk = it % D, rg = it / D;
        const int pdk = perm32(dk);
        uint32_t wv[4];
        if constexpr (IN_F32) {
#pragma unroll
          for (int j = 0; j < 4; ++j) wv[j] = __float_as_uint(sm.kk[E * rg + j][pdk]);
          *reinterpret_cast<uint4 *>(&sm.kt[dk][perm32(E * rg)]) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            wv[j] = (uint32_t)sm.kk[E * rg + 2 * j][pdk] | ((uint32_t)sm.kk[E * rg + 2 * j + 1][pdk] << 16);
          *reinterpret_cast<uint2 *>(&sm.kt[dk][perm32(E * rg)]) = make_uint2(wv[0], wv[1]);
          *reinterpret_cast<uint2 *>(&sm.kt[dk][perm32(E * rg + 4)]) = make_uint2(wv[2], wv[3]);
        }
      }
    } else {
      // channel gate: stage g, prefix-sum each key channel over the chunk;
      // the Gram entries exactly, token pair by token pair; then e^{G} k,
      // e^{G} q and the keys decayed to the chunk's end.
      for (int it = tid; it < C * (BV / 8); it += 256) {
        const int row = it / (BV / 8), c8 = 8 * (it % (BV / 8));
        copy8<IN_F32>(p.v, (t0 + row) * p.v_stride + (int64_t)h * D + vb * BV + c8, row < L,
                      &sm.vv[row][c8]);
      }
      const SubMap map(t0, p.P);   // substeps: the gate on a token's first
      for (int it = tid; it < C * (D / 4); it += 256) {
        const int row = it / (D / 4), c4 = 4 * (it % (D / 4));
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < L && map.sub(row) == 0)
          x = *reinterpret_cast<const float4 *>(p.g + ((map.r0 + map.tok(row)) * p.HV + h) * (int64_t)D + c4);
        *reinterpret_cast<float4 *>(&sm.gstage[row][c4]) = x;
      }
      // raw keys (in kinv) and queries (in qq) for the Gram entries
      for (int it = tid; it < C * (D / 8); it += 256) {
        const int row = it / (D / 8), c8 = 8 * (it % (D / 8));
        const bool ok = row < L;
        float kx[8], qx[8];
        load8<IN_F32>(p.k, (t0 + row) * p.k_stride + (int64_t)hk * D + c8, ok, kx);
        load8<IN_F32>(p.q, (map.r0 + map.tok(row)) * p.q_stride + (int64_t)hk * D + c8, ok, qx);
        *reinterpret_cast<float4 *>(&sm.kinv[row][perm32(c8)]) = make_float4(kx[0], kx[1], kx[2], kx[3]);
        *reinterpret_cast<float4 *>(&sm.kinv[row][perm32(c8 + 4)]) = make_float4(kx[4], kx[5], kx[6], kx[7]);
        *reinterpret_cast<float4 *>(&sm.qq[row][perm32(c8)]) = make_float4(qx[0], qx[1], qx[2], qx[3]);
        *reinterpret_cast<float4 *>(&sm.qq[row][perm32(c8 + 4)]) = make_float4(qx[4], qx[5], qx[6], qx[7]);
      }
      if (w == 0) {
        sm.G[lane] = 0.f;   // decay sits inside the channel-gate operands
        float bl = 0.f;
        if constexpr (DELTA) bl = lane < L ? p.beta[(t0 + lane) * p.HV + h] : 0.f;
        sm.beta[lane] = bl;
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

      // Gram entries of row i = tid / 4 against the 16 keys of column block
      // tid % 4 (lower blocks only): sum_c k_ic k_jc e^{G_ic - G_jc} and
      // sum_c q_ic k_jc e^{G_ic - G_jc} for j <= i, each exponent <= 0, so
      // no decay factor can overflow whatever the gate.
      const int gi = tid >> 2, gjb = tid & 3;
      float racc[16], aacc[16];
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) racc[jj] = aacc[jj] = 0.f;
      if (16 * gjb <= gi) {
        for (int c4 = 0; c4 < D / 4; ++c4) {
          const float4 Gi = *reinterpret_cast<const float4 *>(&sm.gstage[gi][4 * c4]);
          const float4 ki = *reinterpret_cast<const float4 *>(&sm.kinv[gi][perm32(4 * c4)]);
          const float4 qi = *reinterpret_cast<const float4 *>(&sm.qq[gi][perm32(4 * c4)]);
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) {
            const int j = 16 * gjb + jj;
            if (j <= gi) {
              const float4 Gj = *reinterpret_cast<const float4 *>(&sm.gstage[j][4 * c4]);
              const float4 kj = *reinterpret_cast<const float4 *>(&sm.kinv[j][perm32(4 * c4)]);
              const float e0 = __expf(Gi.x - Gj.x), e1 = __expf(Gi.y - Gj.y);
              const float e2 = __expf(Gi.z - Gj.z), e3 = __expf(Gi.w - Gj.w);
              const float t0_ = kj.x * e0, t1_ = kj.y * e1, t2_ = kj.z * e2, t3_ = kj.w * e3;
              if constexpr (DELTA) racc[jj] += ((ki.x * t0_ + ki.y * t1_) + (ki.z * t2_ + ki.w * t3_));
              aacc[jj] += ((qi.x * t0_ + qi.y * t1_) + (qi.z * t2_ + qi.w * t3_));
            }
          }
        }
      }

      // the decayed operands, each thread its own elements: e^{G} k and
      // e^{G} q in place, the keys decayed to the chunk's end kept for the
      // transposed store below
      constexpr int NE = C * D / 256;
      float kend[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int idx = tid + 256 * e, row = idx / D, c = idx % D, pc = perm32(c);
        const float Gv = sm.gstage[row][c], Gl = sm.gstage[C - 1][c];
        const float kr = sm.kinv[row][pc], qr = sm.qq[row][pc];
        const float eg = __expf(Gv);
        sm.kk[row][pc] = kr * eg;
        sm.qq[row][pc] = qr * eg;
        kend[e] = kr * __expf(Gl - Gv);
      }
      __syncthreads();   // raw keys (kinv) and G (gstage) are dead from here on
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int idx = tid + 256 * e;
        sm.kt[idx % D][perm32(idx / D)] = kend[e];
      }
      // Gram entries into the split planes (R's diagonal blocks in fp32)
      if (16 * gjb <= gi) {
        const int I = gi >> 4, r_ = gi & 15;
        const float bi = sm.beta[gi];
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int j = 16 * gjb + jj;
          const float av = j <= gi ? p.scale * aacc[jj] : 0.f;
          store_split(&sm.aqh[0][0], &sm.aql[0][0], gi * SM::PB + j, av);
          if constexpr (DELTA) {
            const float rv = j < gi ? bi * racc[jj] : 0.f;
            if (gjb == I) sm.rd[I][r_][jj] = rv;
            else store_split(&sm.rth[0][0], &sm.rtl[0][0], gi * SM::PB + j, rv);
          }
        }
      }
      __syncthreads();
    }

    // ================= phase 1: Gram matrices (no or scalar gate) =================
    if constexpr (GATE != GDR_GATE_CHANNEL) {
      switch (w) {
        case 0: grams<0, IN_F32, GATE, DELTA, D>(sm, p, r, g); break;
        case 1: grams<1, IN_F32, GATE, DELTA, D>(sm, p, r, g); break;
        case 2: grams<2, IN_F32, GATE, DELTA, D>(sm, p, r, g); break;
        default: grams<3, IN_F32, GATE, DELTA, D>(sm, p, r, g); break;
      }
    }

    // ============ phase 2 (per wave): X = K S^T and Q S^T, eight chains ============
    // They read only keys, queries and this wave's state, so they run before
    // the barrier that publishes the Gram results.
    f32x4 xa[4], qa[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) xa[I] = qa[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      Frag sf;   // state B fragment over key rows 32s .. 32s+31
      chainfrag(st[2 * s], st[2 * s + 1], sf);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        Frag fq;
        ldfrag(&sm.qq[0][0], SM::PK, 16 * I + r, 32 * s, g, fq);
        qa[I] = mm<OPF32, true>(fq, sf, qa[I]);
        if constexpr (DELTA) {
          Frag fk;
          ldfrag(&sm.kk[0][0], SM::PK, 16 * I + r, 32 * s, g, fk);
          xa[I] = mm<OPF32, true>(fk, sf, xa[I]);
        }
      }
    }
    __syncthreads();

    // ======== phase 3: inverses of the diagonal blocks of I + R (wave w: block w) ========
    if constexpr (DELTA) {
      // Forward substitution down the rows of block w (x = column c of T_ww);
      // the four lane groups of a wave solve the same column redundantly
      // (branch free) and each stores a quarter of its rows.
      const int c = lane & 15, q = lane >> 4, o = 16 * w;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float row[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const float4 v4 = *reinterpret_cast<const float4 *>(&sm.rd[w][i][4 * i4]);
          row[4 * i4] = v4.x; row[4 * i4 + 1] = v4.y; row[4 * i4 + 2] = v4.z; row[4 * i4 + 3] = v4.w;
        }
        float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < i; ++j) a4[j & 3] += row[j] * x[j];
        x[i] = ((i == c) ? 1.f : 0.f) - ((a4[0] + a4[1]) + (a4[2] + a4[3]));
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float v = q == 0 ? x[i4] : q == 1 ? x[4 + i4] : q == 2 ? x[8 + i4] : x[12 + i4];
        store_split(&sm.rth[0][0], &sm.rtl[0][0], (o + 4 * q + i4) * SM::PB + o + c, v);
      }
      __syncthreads();
    }

    // ================= phase 4: corrected values, outputs, state (per wave) =================
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
    Frag4 vsp[4];    // their split B fragments
    if constexpr (DELTA) {
      // Vb = (I + R)^-1 R_v by block forward substitution over 16-row blocks:
      // Vb_I = T_II (R_v,I - sum_{J<I} R_IJ Vb_J), with T_II the diagonal
      // inverses and R_IJ the off-diagonal blocks.
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const float4 Bi = *reinterpret_cast<const float4 *>(&sm.beta[16 * I + 4 * g]);
        const float bi[4] = {Bi.x, Bi.y, Bi.z, Bi.w};
        f32x4 rv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = xa[I][i];
          if constexpr (GATE == GDR_GATE_SCALAR) x *= sm.eG[16 * I + 4 * g + i];
          rv[i] = bi[i] * (vt[I][i] - x);
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < I; ++J) {
          Frag4 fr;
          ldsplit4(&sm.rth[0][0], &sm.rtl[0][0], SM::PB, 16 * I + r, 16 * J, g, fr);
          acc = mm16(fr, vsp[J], acc);
        }
        Frag4 fy, ft;
        split4(rv - acc, fy);
        ldsplit4(&sm.rth[0][0], &sm.rtl[0][0], SM::PB, 16 * I + r, 16 * I, g, ft);
        vbar[I] = mm16(ft, fy, f32x4{0.f, 0.f, 0.f, 0.f});
        split4(vbar[I], vsp[I]);
      }
    } else {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        vbar[I] = vt[I];
        split4(vbar[I], vsp[I]);
      }
    }

    // O = s e^{G} (.) Q S^T + A Vb   (A lower triangular: blocks J <= I)
    f32x4 oa[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc = qa[I];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sc = p.scale;
        if constexpr (GATE == GDR_GATE_SCALAR) sc *= sm.eG[16 * I + 4 * g + i];
        acc[i] *= sc;
      }
#pragma unroll
      for (int J = 0; J <= I; ++J) {
        Frag4 fa;
        ldsplit4(&sm.aqh[0][0], &sm.aql[0][0], SM::PB, 16 * I + r, 16 * J, g, fa);
        acc = mm16(fa, vsp[J], acc);
      }
      oa[I] = acc;
    }
    if constexpr (!CKPT) {
      // row (16I + 4g + i) of this chunk, column col: 32-bit offsets from the
      // chunk's first output row
      const uint32_t HVDu = (uint32_t)HVD;
      if (p.P > 1) {
        // substeps: a token's output is its last substep's, at o row
        // (t0 + ii) / P; the other rows are dropped
        const SubMap map(t0, p.P);
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ii = 16 * I + 4 * g + i;
            if (ii < L && map.sub(ii) == map.P - 1) {
              const int64_t off = (map.r0 + map.tok(ii)) * HVD + (int64_t)h * D + col;
              if (p.out_bf16) static_cast<uint16_t *>(p.o)[off] = f32_to_bf16(oa[I][i]);
              else static_cast<float *>(p.o)[off] = oa[I][i];
            }
          }
      } else if (p.out_bf16) {
        uint16_t *ob = static_cast<uint16_t *>(p.o) + t0 * HVD + (int64_t)h * D + col;
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ii = 16 * I + 4 * g + i;
            if (L == C || ii < L) ob[(uint32_t)ii * HVDu] = f32_to_bf16(oa[I][i]);
          }
      } else {
        float *ob = static_cast<float *>(p.o) + t0 * HVD + (int64_t)h * D + col;
        if (L == C) {
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) ob[(uint32_t)(16 * I + 4 * g + i) * HVDu] = oa[I][i];
        } else {
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ii = 16 * I + 4 * g + i;
              if (ii < L) ob[(uint32_t)ii * HVDu] = oa[I][i];
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
        if constexpr (GATE == GDR_GATE_CHANNEL) {
          // S^T <- e^{G_last} (.) S^T + K_end^T Vb (key rows decay first)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[m][i] *= sm.eGlastc[16 * m + 4 * g + i];
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          Frag fa;
          ldfrag(&sm.kt[0][0], SM::PT, 16 * m + r, 32 * s, g, fa);
          st[m] = mm<OPF32, USPLIT>(fa, uf[s], st[m]);
        }
      }
    }
    __syncthreads();   // LDS is rewritten by the next chunk
  }

  // ---- final state back to the pool slot ----
  if constexpr (!CKPT) {
    const int64_t sbase = (slot * p.HV + h) * (int64_t)(D * D) + col;
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
template <bool IN_F32, int GATE, bool DELTA, int D>
hipError_t launch_t(const ChunkParams &p, int N, hipStream_t stream) {
  // one XCD round covers 8 groups of ratio * NB workgroups
  const int grp = p.ratio * (D / BV);
  const int blocks = ((N * p.HK + 7) / 8) * 8 * grp;
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

template <bool IN_F32, int GATE, int D>
hipError_t launch_ckpt(const ChunkParams &p, int N, hipStream_t stream) {
  const int grp = p.ratio * (D / BV);
  const int blocks = ((N * p.HK + 7) / 8) * 8 * grp;
  hipLaunchKernelGGL((chunk_fwd_kernel<IN_F32, GATE, true, D, true>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <bool IN_F32, int GATE>
hipError_t ckpt_by_dim(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.DK == 128) return launch_ckpt<IN_F32, GATE, 128>(p, a.N, s);
  return launch_ckpt<IN_F32, GATE, 64>(p, a.N, s);
}

template <bool IN_F32>
hipError_t ckpt_by_gate(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.gate == GDR_GATE_SCALAR) return ckpt_by_dim<IN_F32, GDR_GATE_SCALAR>(a, p, s);
  return ckpt_by_dim<IN_F32, GDR_GATE_NONE>(a, p, s);
}

}  // namespace

hipError_t launch_chunk_states(const gdr_args &a, float *ckpt, hipStream_t stream) {
  ChunkParams p;
  p.q = a.q; p.k = a.k; p.v = a.v;
  p.q_stride = a.q_stride_t; p.k_stride = a.k_stride_t; p.v_stride = a.v_stride_t;
  p.g = a.g; p.beta = a.beta; p.o = nullptr; p.pool = a.state_pool;
  p.slot_idx = a.slot_idx; p.cu_seqlens = a.cu_seqlens;
  p.N = a.N; p.HK = a.HK; p.HV = a.HV; p.ratio = a.HV / a.HK;
  p.scale = a.scale;
  p.zero_init = (a.flags & GDR_FLAG_ZERO_INIT) ? 1 : 0;
  p.st_bf16 = a.state_dtype == GDR_BF16;
  p.out_bf16 = 0;
  p.P = 1;
  p.rev = 0;
  p.lc = 64;
  p.ckpt = ckpt;
  if (a.in_dtype == GDR_BF16) return ckpt_by_gate<false>(a, p, stream);
  return ckpt_by_gate<true>(a, p, stream);
}

bool prefill_force_generic() {
  static const bool force = [] {
    const char *e = getenv("GDR_PREFILL_KERNEL");
    return e && strcmp(e, "generic") == 0;
  }();
  return force;
}

hipError_t launch_chunk_fwd(const gdr_args &a, hipStream_t stream) {
  // bf16 inputs without a channel gate take the warp-specialised kernel;
  // GDR_PREFILL_KERNEL=generic selects this file's kernel for every case
  // (used to compare them). Chunks of 16 or 32 tokens are this file's kernel.
  if (!prefill_force_generic() && a.in_dtype == GDR_BF16 && a.gate != GDR_GATE_CHANNEL && a.chunk_size == 64)
    return launch_chunk_fwd_ws(a, stream);
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
  p.rev = 0;   // (the reversed walk is the warp-specialised kernel's)
  p.lc = a.chunk_size;
  p.ckpt = nullptr;
  if (a.in_dtype == GDR_BF16) return by_gate<false>(a, p, stream);
  return by_gate<true>(a, p, stream);
}

}  // namespace gdr
