// Types and MFMA helpers shared by the chunk-prefill kernels (gfx950).
// Internal to libgdr.
#pragma once

#include <stdint.h>

#include "gdr_internal.h"

namespace gdr {
namespace chunk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;    // tokens per chunk

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations
// only. __syncthreads also waits for every global load and store in flight
// (vmcnt(0)), which puts a kernel that streams results out behind its own
// stores at each barrier. Global memory written before it is not made
// visible to the other waves. The memory clobbers keep the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// A load through the scalar unit, for data no kernel writes while the
// reader runs (sequence offsets) at a uniform address: it is waited for with
// lgkmcnt, so it does not queue behind the vector loads and stores in flight
// the way a vector load does (their counter drains in order).
__device__ __forceinline__ int32_t scalar_load(const int32_t *ptr) {
  return *(const __attribute__((address_space(4))) int32_t *)ptr;
}
constexpr int BV = 64;   // value columns per workgroup (16 per wave)

// Substep bookkeeping for P transitions per token (Gated DeltaProduct run
// as a virtual sequence): row i of a run of rows that starts at substep t0
// belongs to token r0 + tok(i) and is its substep j0 + i - tok(i) * P.
// tok() divides by P with a 16-bit reciprocal, exact while j0 + i < 4096
// (the rounding error stays below 1/16, and a quotient's fraction is at
// most (P - 1) / P <= 7/8 for P <= 8).
struct SubMap {
  int64_t r0;
  int j0, P, M;
  __device__ __forceinline__ SubMap(int64_t t0, int P_) : P(P_) {
    r0 = t0 / P_;
    j0 = (int)(t0 - r0 * P_);
    M = (65536 + P_ - 1) / P_;
  }
  __device__ __forceinline__ int tok(int i) const { return ((j0 + i) * M) >> 16; }
  __device__ __forceinline__ int sub(int i) const { return j0 + i - tok(i) * P; }
};

struct ChunkParams {
  const void *q, *k, *v;
  int64_t q_stride, k_stride, v_stride;
  const float *g, *beta;
  void *o;
  void *pool;
  const int32_t *slot_idx, *cu_seqlens;
  int32_t N, HK, HV, ratio;
  float scale;
  int zero_init, st_bf16, out_bf16;
  int32_t P;   // transitions per token (Gated DeltaProduct substeps); 1 otherwise
  int32_t rev; // walk each sequence's rows backwards (warp-specialised kernel only)
  int32_t lc;  // tokens per chunk, 16, 32 or 64 (the general kernel; the others take 64)
  float *ckpt; // chunk-start states of the backward's forward walk (general kernel), or NULL
};

__device__ __forceinline__ f32x4 mfma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Frag {
  bf16x8 hi, lo;
};

// Split of two fp32 values into bf16 pairs hi + lo: hi = bf16(x) (nearest
// even, one packed conversion for the pair), lo = bf16(x - hi) of the exact
// fp32 remainder (one more packed conversion). hi + lo carries about 17
// significant bits of the value.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo) {
  const bf16x2 h = {static_cast<__bf16>(x0), static_cast<__bf16>(x1)};
  uint32_t hw = __builtin_bit_cast(uint32_t, h);
  // (the packed pair is made opaque: seen through, the compiler converts x0
  // a second time to shift it into place, one more instruction per pair)
  asm("" : "+v"(hw));
  hi = hw;
  const bf16x2 l = {static_cast<__bf16>(x0 - __uint_as_float(hw << 16)),
                    static_cast<__bf16>(x1 - __uint_as_float(hw & 0xffff0000u))};
  lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ void split8(const float (&x)[8], Frag &f) {
  u32x4 h, l;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t hh, ll;
    split_pair(x[2 * j], x[2 * j + 1], hh, ll);
    h[j] = hh;
    l[j] = ll;
  }
  f.hi = __builtin_bit_cast(bf16x8, h);
  f.lo = __builtin_bit_cast(bf16x8, l);
}

// acc += a * b with the passes the operands need (lo terms first).
template <bool A_SPLIT, bool B_SPLIT>
__device__ __forceinline__ f32x4 mm(const Frag &a, const Frag &b, f32x4 c) {
  if constexpr (A_SPLIT) c = mfma(a.lo, b.hi, c);
  if constexpr (B_SPLIT) c = mfma(a.hi, b.lo, c);
  return mfma(a.hi, b.hi, c);
}

// Pass P of acc += a * b as mm<A_SPLIT, B_SPLIT> issues them (lo terms first,
// then hi x hi; a pass the operands do not need leaves acc as it is). Blocks
// of independent products issue pass by pass across their accumulators, so
// that no MFMA waits on the one just before it; each accumulator still sees
// mm's sequence of products, so results are unchanged.
template <int P, bool A_SPLIT, bool B_SPLIT>
__device__ __forceinline__ f32x4 mm_pass(const Frag &a, const Frag &b, f32x4 c) {
  if constexpr (P == 0) return A_SPLIT ? mfma(a.lo, b.hi, c) : c;
  else if constexpr (P == 1) return B_SPLIT ? mfma(a.hi, b.lo, c) : c;
  else return mfma(a.hi, b.hi, c);
}

// Operand arrays in LDS store each 32-wide block of their contraction axis
// permuted so that a lane's slot set K(g) = {4g..4g+3, 16+4g..16+4g+3} is the
// contiguous physical range 8g .. 8g+7: logical index c sits at perm32(c).
__device__ __forceinline__ int perm32(int c) {
  const int a = (c >> 2) & 7;
  return (c & ~31) + 8 * (a & 3) + 4 * (a >> 2) + (c & 3);
}

// Fragment of row `row`, k step starting at (logical = physical) column col0
// of a permuted operand array: one 16-byte (bf16) or 32-byte (fp32) read.
__device__ __forceinline__ void ldfrag(const uint16_t *base, int pitch, int row, int col0, int g,
                                       Frag &f) {
  const uint4 u = *reinterpret_cast<const uint4 *>(base + row * pitch + col0 + 8 * g);
  f.hi = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void ldfrag(const float *base, int pitch, int row, int col0, int g,
                                       Frag &f) {
  const float *p = base + row * pitch + col0 + 8 * g;
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  split8(x, f);
}

// B fragment over 32 rows built from two stacked accumulator tiles.
__device__ __forceinline__ void chainfrag(const f32x4 &t0, const f32x4 &t1, Frag &f) {
  const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
  split8(x, f);
}

// 16x16x16 products (k = 4g .. 4g+3 per lane): the accumulator layout of a
// 16-row tile is directly a B fragment, so block-triangular chains need no
// reordering.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

struct Frag4 {
  bf16x4 hi, lo;
};

__device__ __forceinline__ f32x4 mfma16(const bf16x4 &a, const bf16x4 &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ void split4(const f32x4 &x, Frag4 &f) {
  uint32_t h0, l0, h1, l1;
  split_pair(x[0], x[1], h0, l0);
  split_pair(x[2], x[3], h1, l1);
  f.hi = __builtin_bit_cast(bf16x4, make_uint2(h0, h1));
  f.lo = __builtin_bit_cast(bf16x4, make_uint2(l0, l1));
}

// acc += a * b, both split (three passes, lo terms first)
__device__ __forceinline__ f32x4 mm16(const Frag4 &a, const Frag4 &b, f32x4 c) {
  c = mfma16(a.lo, b.hi, c);
  c = mfma16(a.hi, b.lo, c);
  return mfma16(a.hi, b.hi, c);
}

// A fragment of a 16x16 block of an fp32 LDS matrix: row `row`, columns
// col0 + 4g .. col0 + 4g + 3.
__device__ __forceinline__ void ldfrag4(const float *base, int pitch, int row, int col0, int g,
                                        Frag4 &f) {
  const float4 a = *reinterpret_cast<const float4 *>(base + row * pitch + col0 + 4 * g);
  const f32x4 x = {a.x, a.y, a.z, a.w};
  split4(x, f);
}


// Split fragment of a 16x16 block of a pre-split bf16 plane pair: row `row`,
// columns col0 + 4g .. col0 + 4g + 3.
__device__ __forceinline__ void ldsplit4(const uint16_t *hi, const uint16_t *lo, int pitch, int row,
                                         int col0, int g, Frag4 &f) {
  const int o = row * pitch + col0 + 4 * g;
  f.hi = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(hi + o));
  f.lo = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2 *>(lo + o));
}

__device__ __forceinline__ void store_split(uint16_t *hi, uint16_t *lo, int idx, float x) {
  const __bf16 h = static_cast<__bf16>(x);
  const __bf16 l = static_cast<__bf16>(x - static_cast<float>(h));
  hi[idx] = __builtin_bit_cast(uint16_t, h);
  lo[idx] = __builtin_bit_cast(uint16_t, l);
}

// Inclusive scan across the 64 lanes of a wave with DPP row shifts and row
// broadcasts (no LDS traffic): shifts 1, 2, 4, 8 scan each row of 16 lanes,
// then lane 15 of row 0/2 is added into row 1/3 and lane 31 into rows 2-3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  const int s = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf, false);
  return v + __builtin_bit_cast(float, s);
}

__device__ __forceinline__ float wave_scan_dpp(float x) {
  x = dpp_add<0x111, 0xf>(x);   // row_shr:1
  x = dpp_add<0x112, 0xf>(x);   // row_shr:2
  x = dpp_add<0x114, 0xf>(x);   // row_shr:4
  x = dpp_add<0x118, 0xf>(x);   // row_shr:8
  x = dpp_add<0x142, 0xa>(x);   // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Lane J of every row of 16 lanes, broadcast to that row (DPP row_newbcast;
// every lane is written, so no old value is needed).
template <int J>
__device__ __forceinline__ float row_bcast16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J, 0xf, 0xf, false));
}

// Right-looking substitution for the inverse of a unit lower triangular
// 16x16 matrix I + N (N strictly lower, exact zeros on and above the
// diagonal). Lane (r, g) holds row r of -N in nn[] and row r, columns
// 4g .. 4g+3 of the inverse in t[] (start: row r of I). At step J row J of
// the inverse is final; every row r adds -N[r][J] times it. One instruction
// per step and column: v_fmac_f32 with its first source broadcast from lane J
// of each row of 16 by DPP. Three instructions separate a write of t[i] from
// the next step's DPP read of it (two wait states are required), and the
// leading s_nop covers the values written before the sequence.
#define GDR_INV_STEP(J)                                                                            \
  "v_fmac_f32_dpp %0, %0, %[n" #J "] row_newbcast:" #J " row_mask:0xf bank_mask:0xf\n"          \
  "v_fmac_f32_dpp %1, %1, %[n" #J "] row_newbcast:" #J " row_mask:0xf bank_mask:0xf\n"          \
  "v_fmac_f32_dpp %2, %2, %[n" #J "] row_newbcast:" #J " row_mask:0xf bank_mask:0xf\n"          \
  "v_fmac_f32_dpp %3, %3, %[n" #J "] row_newbcast:" #J " row_mask:0xf bank_mask:0xf\n"
__device__ __forceinline__ void unit_lower_inverse16(float (&t)[4], const float (&nn)[16]) {
  asm volatile("s_nop 1\n" GDR_INV_STEP(0) GDR_INV_STEP(1) GDR_INV_STEP(2) GDR_INV_STEP(3)
               GDR_INV_STEP(4) GDR_INV_STEP(5) GDR_INV_STEP(6) GDR_INV_STEP(7) GDR_INV_STEP(8)
               GDR_INV_STEP(9) GDR_INV_STEP(10) GDR_INV_STEP(11) GDR_INV_STEP(12) GDR_INV_STEP(13)
               GDR_INV_STEP(14) GDR_INV_STEP(15)
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3])
               : [n0] "v"(nn[0]), [n1] "v"(nn[1]), [n2] "v"(nn[2]), [n3] "v"(nn[3]),
                 [n4] "v"(nn[4]), [n5] "v"(nn[5]), [n6] "v"(nn[6]), [n7] "v"(nn[7]),
                 [n8] "v"(nn[8]), [n9] "v"(nn[9]), [n10] "v"(nn[10]), [n11] "v"(nn[11]),
                 [n12] "v"(nn[12]), [n13] "v"(nn[13]), [n14] "v"(nn[14]), [n15] "v"(nn[15]));
}
#undef GDR_INV_STEP

__device__ __forceinline__ float lane_value(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// Sum over the four 16-lane rows of the wave (the same lane of each), with
// gfx950's lane swaps: permlane16_swap exchanges the odd 16-lane rows of its
// first operand with the even rows of its second, permlane32_swap the upper
// half of the first with the lower half of the second; with x in both, every
// lane receives its partner's x beside its own.
__device__ __forceinline__ float sum_lane_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

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

// (Vector types, not arrays: prefetched data stays in registers as SSA values.)
template <int N>
struct U32Vec {
  typedef unsigned int type __attribute__((ext_vector_type(N)));
};

template <class Vec>
__device__ __forceinline__ void put4(Vec &v, int u, const uint4 x) {
  v[4 * u] = x.x; v[4 * u + 1] = x.y; v[4 * u + 2] = x.z; v[4 * u + 3] = x.w;
}
template <class Vec>
__device__ __forceinline__ uint4 get4(const Vec &v, int u) {
  return make_uint4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]);
}


// Scheduling hint for the block that follows the code it is placed after:
// N times, one MFMA followed by up to V VALU and R LDS-read instructions, so
// that independent vector work and loads issue while the products run.
template <int N, int V, int R>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x002, V, 0);
    if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  }
}

// Bound of every wait on an LDS counter. A wait that runs out goes on with
// whatever the counter's producers have stored by then, so it cannot hang;
// it also sets g_wait_timeout, which the host clears before and reads after
// a call made with GDR_FLAG_DEBUG_CHECKS and reports as GDR_E_DEVICE_CHECK.
// (A wait runs out only if a producer wave never signals: a defect, never a
// matter of timing; 2^20 polls with a sleep each last well over 10 ms.)
constexpr int SPIN = 1 << 20;

// One word per translation unit that includes this header.
static __device__ int g_wait_timeout;

__device__ __forceinline__ void note_wait_timeout() {
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(&g_wait_timeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void spin_until(const int *ctr, int target) {
  // an LDS-typed pointer: a generic one compiles to a flat load, which would
  // also wait for global loads in flight
  typedef __attribute__((address_space(3))) volatile int lds_vint;
  const lds_vint *p = (const lds_vint *)ctr;
  bool done = false;
  for (int spin = 0; spin < SPIN; ++spin) {
    if (*p >= target) {
      done = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (!done) note_wait_timeout();
  asm volatile("" ::: "memory");
}

// Host side of g_wait_timeout for the including translation unit: clear it
// (clear = true) or copy it to *out, both enqueued on `stream`.
static inline hipError_t wait_flag_access(int *out, bool clear, hipStream_t stream) {
  static const int zero = 0;
  if (clear) return hipMemcpyToSymbolAsync(HIP_SYMBOL(g_wait_timeout), &zero, sizeof(int), 0,
                                           hipMemcpyHostToDevice, stream);
  return hipMemcpyFromSymbolAsync(out, HIP_SYMBOL(g_wait_timeout), sizeof(int), 0, hipMemcpyDeviceToHost,
                                  stream);
}

// This wave's LDS stores land, then one lane counts the wave in.
__device__ __forceinline__ void count_in(int *ctr, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) atomicAdd(ctr, 1);
}
__device__ __forceinline__ void count_in(int *ctr0, int *ctr1, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) {
    atomicAdd(ctr0, 1);
    atomicAdd(ctr1, 1);
  }
}

// Fragment of a transposed operand read from a token-major bf16 array with
// two transposing reads (ds_read_b64_tr_b16): M rows are 16 columns of the
// array, K the tokens of k step s in slot order K(g). Within each 16-lane
// group the read hands lane i, slot j element (i mod 4) of the 4 elements
// addressed by lane 4j + i/4; lane a therefore addresses token
// 32s + 4g + a/4 (+16 for the second half) at the four consecutive array
// columns that start at physical column `col4` (the group of logical columns
// 16m + 4 (a mod 4) .. +3 of the tile).
__device__ __forceinline__ void ldfrag_tr(const uint16_t *kk, int pitch, int col4, int s, int r, int g,
                                          Frag &f) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const uint16_t *p0 = kk + (32 * s + 4 * g + (r >> 2)) * pitch + col4;
  const uint16_t *p1 = p0 + 16 * pitch;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  f.hi = __builtin_bit_cast(bf16x8, ab);
}

// K^T fragment for the state update: key rows 16m .. 16m+15 (M), tokens of
// k step s (K), from the token-major key array whose columns are permuted
// (perm32).
__device__ __forceinline__ void ldfrag_kt(const uint16_t *kk, int pitch, int m, int s, int r, int g,
                                          Frag &f) {
  ldfrag_tr(kk, pitch, perm32(16 * m + 4 * (r & 3)), s, r, g, f);
}

}  // namespace chunk

hipError_t launch_chunk_fwd_ws(const gdr_args &a, hipStream_t stream);

}  // namespace gdr
