// Warp-specialised chunkwise prefill (bf16 q/k/v, no gate or a scalar gate).
//
// Same mathematics as chunk_fwd.hip (section 6 of "You Could Have Come Up With
// Kimi Delta Attention"; section 4 of "From Attention to Learned Memory"), but
// the work of a chunk is split between two groups of waves that run
// concurrently on every SIMD:
//
//   * state waves 0-3 own 16 value columns each (state S^T[DK, 16] resident in
//     MFMA accumulators) and do everything that depends on the state for
//     chunk c: X = K S^T, Q S^T, the block triangular solve of the corrected
//     values, the outputs and the state update;
//   * prep waves 4-7 do everything that does not, one chunk ahead: write
//     chunk c+1's keys and queries into LDS (from registers loaded one more
//     chunk ahead), the gate prefix sums, the Gram matrices R and A, and the
//     16x16 diagonal inverses of I + R (in registers, by the waves that
//     formed those blocks of R).
//
// Keys, queries, the coefficient planes and the gate factors are double
// buffered in LDS (set c % 2 is read by the state waves while the prep waves
// fill set (c+1) % 2), so one workgroup barrier per chunk suffices. The prep
// waves synchronise among themselves through an LDS counter: their key and
// query stores must land before their Gram matrices read them.
//
// The state update reads K^T fragments straight from the token-major key
// array with the transposing LDS read of gfx950 (ds_read_b64_tr_b16), so no
// transposed copy of the keys is kept.
#include "chunk_common.h"

namespace gdr {
namespace {

using namespace chunk;

constexpr int NTH = 512;   // 8 waves

template <int D>
struct SmemWS {
  static constexpr int PK = D + 8;   // bf16 token-major rows (permuted k blocks)
  static constexpr int PB = C + 8;   // bf16 C x C planes
  struct Set {
    uint16_t kk[C][PK];
    uint16_t qq[C][PK];
    uint16_t rth[C][PB], rtl[C][PB];   // R off-diagonal blocks, T_II on the diagonal
    uint16_t aqh[C][PB], aql[C][PB];   // A
    float G[C], eG[C], eGl[C], beta[C];
    float eGlast, pad_[3];
  };
  Set set[2];
  float rd[4][16][20];   // R's diagonal blocks in fp32, each read back only by the wave that wrote it
  uint16_t vx[4][C][16];  // per state wave: its 16 value columns of the chunk, token-major (swizzled halves)
  int kcount;            // prep-wave store counter (monotonic)
};

// Prep-wave registers for one chunk's keys, queries and gates.
template <int D>
struct PrefWS {
  static constexpr int KU = C * D / 8 / 256;   // 16-byte units per prep thread
  typename U32Vec<4 * KU>::type k, q;
  float g, beta;
};

template <int GATE, bool DELTA, int D>
__device__ __forceinline__ void prep_load(PrefWS<D> &pf, const ChunkParams &p, int64_t t0, int L,
                                          int h, int hk, int ptid) {
  constexpr int KU = PrefWS<D>::KU;
  const int krow = ptid / (D / 8), krs = 256 / (D / 8), kc = (ptid % (D / 8)) * 16;
  const char *kb = static_cast<const char *>(p.k) + (t0 * p.k_stride + (int64_t)hk * D) * 2;
  const char *qb = static_cast<const char *>(p.q) + (t0 * p.q_stride + (int64_t)hk * D) * 2;
  const uint32_t ks = (uint32_t)(p.k_stride * 2), qs = (uint32_t)(p.q_stride * 2);
  const int last = L - 1;
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
}

// Gram matrices of one chunk (see grams() in chunk_fwd.hip for the tile
// assignment): tile (I, J) is computed transposed so that a lane holds row
// ii = 16I + r, columns 16J + 4g .. +3, stored as split bf16 planes. R's
// diagonal blocks are replaced by their unit lower triangular inverses.
template <int W, int GATE, bool DELTA, int D, class Set>
__device__ __forceinline__ void grams_ws(Set &S, float (*rd)[16][20], float scale, int r, int g,
                                         int pitch_k, int pitch_b) {
  constexpr int NS = D / 32;
  constexpr bool ISQ = DELTA ? (W >= 2) : true;
  constexpr int IA = DELTA ? (W & 1) : W;
  constexpr int NRB = DELTA ? 2 : 1;
  constexpr int IB = DELTA ? 3 - IA : IA;
  constexpr int JMAX = IB > IA ? IB : IA;
  const uint16_t *nrow = ISQ ? &S.qq[0][0] : &S.kk[0][0];

  Frag fn[NRB][NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    ldfrag(nrow, pitch_k, 16 * IA + r, 32 * s, g, fn[0][s]);
    if constexpr (DELTA) ldfrag(nrow, pitch_k, 16 * IB + r, 32 * s, g, fn[NRB - 1][s]);
  }
  f32x4 acc[NRB][4];
#pragma unroll
  for (int J = 0; J <= JMAX; ++J) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) acc[rb][J] = f32x4{0.f, 0.f, 0.f, 0.f};
    Frag fm[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) ldfrag(&S.kk[0][0], pitch_k, 16 * J + r, 32 * s, g, fm[s]);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int I = rb ? IB : IA;
      if (J <= I) {
#pragma unroll
        for (int s = 0; s < NS; ++s) acc[rb][J] = mm<false, false>(fm[s], fn[rb][s], acc[rb][J]);
      }
    }
  }
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int I = rb ? IB : IA;
    const int ii = 16 * I + r;
    const float Gi = S.G[ii], bi = S.beta[ii];
#pragma unroll
    for (int J = 0; J <= I; ++J) {
      const float4 Gj4 = *reinterpret_cast<const float4 *>(&S.G[16 * J + 4 * g]);
      const float Gj[4] = {Gj4.x, Gj4.y, Gj4.z, Gj4.w};
      float val[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jj = 16 * J + 4 * g + i;
        float gam = 1.f;
        if constexpr (GATE == GDR_GATE_SCALAR) gam = __expf(Gi - Gj[i]);
        if constexpr (ISQ) val[i] = (jj <= ii) ? scale * acc[rb][J][i] * gam : 0.f;
        else val[i] = (jj < ii) ? bi * acc[rb][J][i] * gam : 0.f;
      }
      if (!ISQ && J == I) {
        *reinterpret_cast<float4 *>(&rd[I][r][4 * g]) = make_float4(val[0], val[1], val[2], val[3]);
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
        uint16_t *ph = ISQ ? &S.aqh[0][0] : &S.rth[0][0];
        uint16_t *pl = ISQ ? &S.aql[0][0] : &S.rtl[0][0];
        *reinterpret_cast<uint2 *>(ph + ii * pitch_b + 16 * J + 4 * g) = hw;
        *reinterpret_cast<uint2 *>(pl + ii * pitch_b + 16 * J + 4 * g) = lw;
      }
    }
  }
  if constexpr (!ISQ) {
    // T_II = (I + R_II)^{-1} in registers; rd[I] (this wave's own rows)
    // hands every lane its full row of R_II
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int I = rb ? IB : IA;
      float nrow[16], t[4];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 v4 = *reinterpret_cast<const float4 *>(&rd[I][r][4 * i4]);
        nrow[4 * i4] = v4.x; nrow[4 * i4 + 1] = v4.y; nrow[4 * i4 + 2] = v4.z; nrow[4 * i4 + 3] = v4.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] = (r == 4 * g + i) ? 1.f : 0.f;
      unit_lower_inverse16<0>(t, nrow);
      uint16_t hb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 hh = static_cast<__bf16>(t[i]);
        hb[i] = __builtin_bit_cast(uint16_t, hh);
        lb[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(t[i] - static_cast<float>(hh)));
      }
      const int idx = (16 * I + r) * pitch_b + 16 * I + 4 * g;
      *reinterpret_cast<uint2 *>(&S.rth[0][0] + idx) =
          make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
      *reinterpret_cast<uint2 *>(&S.rtl[0][0] + idx) =
          make_uint2(lb[0] | ((uint32_t)lb[1] << 16), lb[2] | ((uint32_t)lb[3] << 16));
    }
  }
}

// K^T fragment for the state update: key rows 16m .. 16m+15 (M), tokens of
// k step s in slot order K(g) (K), read from the token-major key array with
// two transposing reads. Within each 16-lane group the read hands lane i,
// slot j element (i mod 4) of the 4 elements addressed by lane 4j + i/4;
// lane a therefore addresses token 32s + 4g + a/4 (+16 for the second half),
// key columns 16m + 4 (a mod 4) .. +3.
__device__ __forceinline__ void ldfrag_kt(const uint16_t *kk, int pitch, int m, int s, int r, int g,
                                          Frag &f) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int col = perm32(16 * m + 4 * (r & 3));
  const uint16_t *p0 = kk + (32 * s + 4 * g + (r >> 2)) * pitch + col;
  const uint16_t *p1 = p0 + 16 * pitch;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  f.hi = __builtin_bit_cast(bf16x8, ab);
}

// Prep role (waves 4-7): stages chunk c+1 while the state waves run chunk c.
template <int GATE, bool DELTA, int D>
__device__ __forceinline__ void chunk_prep_role(const ChunkParams &p, SmemWS<D> &sm, int pw, int ptid,
                                                int lane, int r, int g, int h, int hk, int64_t bos,
                                                int64_t eos, int nc) {
  using SM = SmemWS<D>;
  using PF = PrefWS<D>;
  constexpr int PK = SM::PK, PB = SM::PB;
  PF pf;
  pf.g = pf.beta = 0.f;
  // work for chunk ci into set ci % 2
  auto prep = [&](int ci) {
    auto &S = sm.set[ci & 1];
    const int64_t t0 = bos + (int64_t)ci * C;
    const int L = (int)min<int64_t>(C, eos - t0);
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int krow = ptid / (D / 8), krs = 256 / (D / 8), c8 = 8 * (ptid % (D / 8));
#pragma unroll
    for (int u = 0; u < PF::KU; ++u) {
      const int row = krow + u * krs;
      const bool ok = row < L;
      const uint4 kx = ok ? get4(pf.k, u) : z, qx = ok ? get4(pf.q, u) : z;
      *reinterpret_cast<uint2 *>(&S.kk[row][perm32(c8)]) = make_uint2(kx.x, kx.y);
      *reinterpret_cast<uint2 *>(&S.kk[row][perm32(c8 + 4)]) = make_uint2(kx.z, kx.w);
      *reinterpret_cast<uint2 *>(&S.qq[row][perm32(c8)]) = make_uint2(qx.x, qx.y);
      *reinterpret_cast<uint2 *>(&S.qq[row][perm32(c8 + 4)]) = make_uint2(qx.z, qx.w);
    }
    if (pw == 0) {
      const bool ok = lane < L;
      float gl = 0.f;
      if constexpr (GATE == GDR_GATE_SCALAR) gl = ok ? pf.g : 0.f;
      const float Gi = wave_scan_dpp(gl);
      const float Gl = lane_value(Gi, 63);
      S.G[lane] = Gi;
      S.eG[lane] = __expf(Gi);
      S.eGl[lane] = __expf(Gl - Gi);
      if (lane == 0) S.eGlast = __expf(Gl);
      S.beta[lane] = ok ? pf.beta : 0.f;
    }
    if (ci + 1 < nc) {
      const int64_t tn = t0 + C;
      prep_load<GATE, DELTA, D>(pf, p, tn, (int)min<int64_t>(C, eos - tn), h, hk, ptid);
    }
    // all prep waves' key/query stores land before any prep wave reads them:
    // wait for this wave's LDS stores only (the prefetch stays in flight),
    // then count in and spin on the counter (bounded)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) atomicAdd(&sm.kcount, 1);
    // an LDS-typed pointer: a generic one compiles to a flat load, which
    // would also wait for the prefetch in flight
    typedef __attribute__((address_space(3))) volatile int lds_vint;
    const lds_vint *kcount_lds = (const lds_vint *)&sm.kcount;
    const int target = 4 * ci + 4;
    for (int spin = 0; spin < (1 << 24); ++spin) {
      if (*kcount_lds >= target) break;
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
    switch (pw) {
      case 0: grams_ws<0, GATE, DELTA, D>(S, sm.rd, p.scale, r, g, PK, PB); break;
      case 1: grams_ws<1, GATE, DELTA, D>(S, sm.rd, p.scale, r, g, PK, PB); break;
      case 2: grams_ws<2, GATE, DELTA, D>(S, sm.rd, p.scale, r, g, PK, PB); break;
      default: grams_ws<3, GATE, DELTA, D>(S, sm.rd, p.scale, r, g, PK, PB); break;
    }
  };

  if (nc == 0) return;
  prep_load<GATE, DELTA, D>(pf, p, bos, (int)min<int64_t>(C, eos - bos), h, hk, ptid);
  prep(0);
  __syncthreads();   // chunk 0 staged
  for (int c = 0; c < nc; ++c) {
    if (c + 1 < nc) prep(c + 1);
    __syncthreads();   // set c % 2 is free again once the state waves are done with it
  }
}

template <int GATE, bool DELTA, int D>
__global__ __launch_bounds__(NTH) void chunk_fwd_ws_kernel(ChunkParams p) {
  using SM = SmemWS<D>;
  constexpr int NB = D / BV;
  constexpr int NT = D / 16;
  constexpr int NS = D / 32;
  constexpr int PK = SM::PK, PB = SM::PB;
  __shared__ SM sm;

  // XCD-aware decomposition (see chunk_fwd.hip)
  const int GRP = p.ratio * NB;
  const int b = blockIdx.x;
  const int gi = (b / (8 * GRP)) * 8 + (b & 7);
  if (gi >= p.N * p.HK) return;
  const int j = (b >> 3) % GRP;
  const int n = gi / p.HK;
  const int hk = gi - n * p.HK;
  const int h = hk * p.ratio + j / NB;
  const int vb = j % NB;

  const int tid = threadIdx.x;
  const int lane = tid & 63, r = lane & 15, g = lane >> 4;
  // the wave index through readfirstlane is provably uniform, so the role
  // branch below is a scalar branch and each role runs its own loop
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bos = p.cu_seqlens[n], eos = p.cu_seqlens[n + 1];
  const int nc = (int)((eos - bos + C - 1) / C);
  const int64_t HVD = (int64_t)p.HV * D;
  if (tid == 0) sm.kcount = 0;
  __syncthreads();   // kcount initialised

  // Both roles pass the same barriers: one after the prologue and one at the
  // end of every chunk (nc + 1 in all when nc > 0, none when nc == 0).
  if (w >= 4) {
    chunk_prep_role<GATE, DELTA, D>(p, sm, w - 4, tid - 256, lane, r, g, h, hk, bos, eos, nc);
    return;
  }

  // state waves: this lane's value column and resident state
  const int col = vb * BV + 16 * w + r;
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
  auto load_v = [&](int ci) {
    const int64_t t0 = bos + (int64_t)ci * C;
    const int last = (int)min<int64_t>(C, eos - t0) - 1;
    const char *vbase = static_cast<const char *>(p.v) + (t0 * p.v_stride + (int64_t)h * D + vb * BV + 16 * w) * 2;
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
    {
      const auto &S = sm.set[c & 1];
      const int64_t t0 = bos + (int64_t)c * C;
      const int L = (int)min<int64_t>(C, eos - t0);

      // this chunk's values, then the next chunk's loads go in flight
      // Token-major values go through this wave's LDS tile (16-byte halves
      // swapped on rows with bit 3 set, so the row writes do not collide) and
      // come back in the accumulator layout: lane (r, g), slot i of block I
      // holds V[16I + 4g + i][r]. Tokens past the sequence end are zero.
      f32x4 vt[4];
      {
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        uint16_t *vx = &sm.vx[w][0][0];
        const uint4 z = make_uint4(0, 0, 0, 0);
        const bool okv = lane < L;
        const int sw = (lane >> 3) & 1;
        *reinterpret_cast<uint4 *>(vx + lane * 16 + 8 * sw) = okv ? get4(vreg, 0) : z;
        *reinterpret_cast<uint4 *>(vx + lane * 16 + 8 * (sw ^ 1)) = okv ? get4(vreg, 1) : z;
        if (c + 1 < nc) load_v(c + 1);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const int row = 16 * I + 4 * g + (r >> 2);
          const int half = ((r & 3) >> 1) ^ ((row >> 3) & 1);
          const s16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4 *)(vx + row * 16 + 8 * half + 4 * (r & 1)));
#pragma unroll
          for (int i = 0; i < 4; ++i) vt[I][i] = bf16_to_f32((uint16_t)t[i]);
        }
      }

      // X = K S^T (delta rule) and Q S^T
      f32x4 xa[4], qa[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) xa[I] = qa[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Frag sf;
        chainfrag(st[2 * s], st[2 * s + 1], sf);
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          Frag fq;
          ldfrag(&S.qq[0][0], PK, 16 * I + r, 32 * s, g, fq);
          qa[I] = mm<false, true>(fq, sf, qa[I]);
          if constexpr (DELTA) {
            Frag fk;
            ldfrag(&S.kk[0][0], PK, 16 * I + r, 32 * s, g, fk);
            xa[I] = mm<false, true>(fk, sf, xa[I]);
          }
        }
      }

      f32x4 vbar[4];
      Frag4 vsp[4];
      if constexpr (DELTA) {
        // Vb_I = T_II (beta (V - e^{G} X)_I - sum_{J<I} R_IJ Vb_J)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const float4 Bi = *reinterpret_cast<const float4 *>(&S.beta[16 * I + 4 * g]);
          const float4 Ei = *reinterpret_cast<const float4 *>(&S.eG[16 * I + 4 * g]);
          const float bi[4] = {Bi.x, Bi.y, Bi.z, Bi.w}, ei[4] = {Ei.x, Ei.y, Ei.z, Ei.w};
          f32x4 rv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = xa[I][i];
            if constexpr (GATE == GDR_GATE_SCALAR) x *= ei[i];
            rv[i] = bi[i] * (vt[I][i] - x);
          }
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int J = 0; J < I; ++J) {
            Frag4 fr;
            ldsplit4(&S.rth[0][0], &S.rtl[0][0], PB, 16 * I + r, 16 * J, g, fr);
            acc = mm16(fr, vsp[J], acc);
          }
          Frag4 fy, ft;
          split4(rv - acc, fy);
          ldsplit4(&S.rth[0][0], &S.rtl[0][0], PB, 16 * I + r, 16 * I, g, ft);
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

      // O = s e^{G} (.) Q S^T + A Vb
      f32x4 oa[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = qa[I];
        const float4 Ei = *reinterpret_cast<const float4 *>(&S.eG[16 * I + 4 * g]);
        const float ei[4] = {Ei.x, Ei.y, Ei.z, Ei.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sc = p.scale;
          if constexpr (GATE == GDR_GATE_SCALAR) sc *= ei[i];
          acc[i] *= sc;
        }
#pragma unroll
        for (int J = 0; J <= I; ++J) {
          Frag4 fa;
          ldsplit4(&S.aqh[0][0], &S.aql[0][0], PB, 16 * I + r, 16 * J, g, fa);
          acc = mm16(fa, vsp[J], acc);
        }
        oa[I] = acc;
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
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int srow = (16 * I + i) * (int)orow;
            const bool ok = L == C || 16 * I + 4 * g + i < L;
            if (p.out_bf16) {
              if (ok) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(oa[I][i]), ors, olane, srow, 0);
            } else {
              if (ok) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(oa[I][i]), ors, olane, srow, 0);
            }
          }
      }

      // S^T <- e^{G_last} S^T + K^T (e^{G_last - G_j} Vb_j)
      {
        f32x4 vs[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const float4 El = *reinterpret_cast<const float4 *>(&S.eGl[16 * I + 4 * g]);
          const float el[4] = {El.x, El.y, El.z, El.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = vbar[I][i];
            if constexpr (GATE == GDR_GATE_SCALAR) x *= el[i];
            vs[I][i] = x;
          }
        }
        Frag uf[2];
        chainfrag(vs[0], vs[1], uf[0]);
        chainfrag(vs[2], vs[3], uf[1]);
        if constexpr (GATE == GDR_GATE_SCALAR) {
          const float a = S.eGlast;
#pragma unroll
          for (int m = 0; m < NT; ++m) st[m] *= a;
        }
        constexpr bool USPLIT = DELTA || GATE == GDR_GATE_SCALAR;
#pragma unroll
        for (int m = 0; m < NT; ++m) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            Frag fa;
            ldfrag_kt(&S.kk[0][0], PK, m, s, r, g, fa);
            st[m] = mm<false, USPLIT>(fa, uf[s], st[m]);
          }
        }
      }
    }
    __syncthreads();   // set c % 2 is refilled by the prep waves next
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

template <int GATE, bool DELTA, int D>
hipError_t launch_ws(const ChunkParams &p, hipStream_t stream) {
  const int grp = p.ratio * (D / BV);
  const int blocks = ((p.N * p.HK + 7) / 8) * 8 * grp;
  hipLaunchKernelGGL((chunk_fwd_ws_kernel<GATE, DELTA, D>), dim3(blocks), dim3(NTH), 0, stream, p);
  return hipGetLastError();
}

template <int GATE, bool DELTA>
hipError_t ws_by_dim(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.DK == 128) return launch_ws<GATE, DELTA, 128>(p, s);
  return launch_ws<GATE, DELTA, 64>(p, s);
}

template <int GATE>
hipError_t ws_by_rule(const gdr_args &a, const ChunkParams &p, hipStream_t s) {
  if (a.rule == GDR_RULE_DELTA) return ws_by_dim<GATE, true>(a, p, s);
  return ws_by_dim<GATE, false>(a, p, s);
}

}  // namespace

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
  if (a.gate == GDR_GATE_SCALAR) return ws_by_rule<GDR_GATE_SCALAR>(a, p, stream);
  return ws_by_rule<GDR_GATE_NONE>(a, p, stream);
}

}  // namespace gdr
