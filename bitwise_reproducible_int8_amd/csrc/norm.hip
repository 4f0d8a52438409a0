// norm.hip -- fixed-order RMSNorm (forward, backward) and the global
// gradient norm (Open-1B report §3.1 "RMSNorm": pre-norm, no bias; FP32
// normalisation; §3.2 "Optimizer": clipping at global l2 norm 1.0, with
// FP32 gradient reduction).
//
// Row sums use the canonical pairwise tree over the row's D leaves: vector
// v of the row is an aligned run whose lanes pair up through the wave
// butterfly (and, for the backward's 4-wave rows, one LDS step), then the
// vectors' nodes pair up in registers.  Columns past D are +0 (forward,
// non-negative leaves) or -0 (backward, signed leaves): both are exact
// additive identities there, i.e. the "unpaired node moves up" rule.
//
// The backward's dg[j] is a tree over tokens.  Each work-group owns R
// consecutive (aligned) tokens and folds its rows, in token order, with a
// binary-carry stack per column: pushing row t merges ctz(t+1) pending
// nodes, lower tokens always on the left, which is exactly node(log2 R, .)
// of the token tree.  Fold kernels then combine those per-block nodes 32 at
// a time with the same stack, padding past the last block with -0, until one
// node per column remains.
#include <string.h>

#include "device.hpp"
#include "internal.hpp"

namespace brq {

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <typename T>
__device__ __forceinline__ u32x4 pack_out(const float* y);
template <>
__device__ __forceinline__ u32x4 pack_out<uint16_t>(const float* y) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(y[2 * i], y[2 * i + 1]);
  return u32x4{w[0], w[1], w[2], w[3]};
}
template <>
__device__ __forceinline__ u32x4 pack_out<float>(const float* y) {
  return u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
               __float_as_uint(y[3])};
}

// DAZ of 8 bf16 values (two per 32-bit word: a half whose exponent field is
// zero keeps only its sign), their exact widening to binary32, and the
// biased exponent of the smallest nonzero value (512 when all are zero).
// Packed 16-bit operations: per word one mask, two for the DAZ, two for the
// exponent minimum.
__device__ __forceinline__ int widen_bf16x8_daz(u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  u16x2_t emin = {0xffff, 0xffff};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = bf16x2_daz(w[i]);
    f[2 * i] = __uint_as_float(u << 16);
    f[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
    // (E - 1) << 7 for E >= 1; a zero exponent wraps to 0xff80
    const u16x2_t th = __builtin_bit_cast(u16x2_t, w[i] & 0x7f807f80u);
    emin = __builtin_elementwise_min(emin, th - u16x2_t{0x80, 0x80});
  }
  const uint32_t lo = emin.x, hi = emin.y;
  return (int)((lo < hi ? lo : hi) >> 7) + 1;
}

// biased exponent of a binary32 value's magnitude
__device__ __forceinline__ int f32_exp(float v) { return (int)((__float_as_uint(v) >> 23) & 0xffu); }

// ---- forward: one wave per row, 4 rows per work-group ------------------------
template <typename T, int V>
__global__ __launch_bounds__(256) void k_rms_fwd(const T* __restrict__ x, const T* __restrict__ g,
                                                 int64_t Tn, int64_t D, float invD, float eps,
                                                 T* __restrict__ y, float* __restrict__ rstd,
                                                 int32_t* flags) {
  constexpr int E = Elem<T>::kPerVec;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= Tn) return;
  const T* xr = x + row * D;
  // bf16 rows skip the flushes where exponent bounds prove them identities
  // (the argument of the backward's unflushed form): with Ex the biased
  // exponent of the wave's smallest nonzero x (after DAZ), every square is
  // at least 2^(2 Ex - 254), normal when Ex >= 64; with Er of rstd and Eg
  // of the lane's smallest nonzero g, x r >= 2^(Ex + Er - 254) and
  // (x r) g >= 2^(Ex + Er + Eg - 381), normal when Ex + Er >= 128 and
  // Ex + Er + Eg >= 255.  Sums of normal non-negative squares are never
  // subnormal.
  constexpr bool kSpec = E == 8;
  float f[V][E];
  int ex = 512;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    const u32x4 raw = c0 < D ? ld16(xr + c0) : u32x4{0, 0, 0, 0};
    if constexpr (kSpec) {
      const int e = widen_bf16x8_daz(raw, f[v]);
      ex = e < ex ? e : ex;
    } else {
      Elem<T>::unpack(raw, f[v]);
    }
  }
  const bool sq_fast = kSpec && __ballot(ex < 64) == 0;
  float node[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float sq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) sq[e] = sq_fast ? f[v][e] * f[v][e] : flush_nonneg(f[v][e] * f[v][e]);
    node[v] = wave_tree<false>(reg_tree<false, E>(sq));
  }
  const float ss = reg_tree<false, V>(node);
  const float ms = fmul(ss, invD);
  const float r = fl_div(1.0f, fl_sqrt(fadd(ms, eps)));
  const int er = f32_exp(r);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    float gv[E], o[E];
    bool fast = false;
    const u32x4 graw = c0 < D ? ld16(g + c0) : u32x4{0, 0, 0, 0};
    if constexpr (kSpec) {
      const int eg = widen_bf16x8_daz(graw, gv);
      fast = __ballot(c0 < D && (ex + er < 128 || ex + er + eg < 255)) == 0;
    } else {
      Elem<T>::unpack(graw, gv);
    }
    if (fast) {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = (f[v][e] * r) * gv[e];
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = fmul(fmul(f[v][e], r), gv[e]);
    }
    if (c0 < D) st16(y + row * D + c0, pack_out<T>(o));
  }
  if (lane == 0) {
    rstd[row] = r;
    if (!__builtin_isfinite(ss)) set_flag(flags, BRQ_FLAG_NONFINITE);
  }
}

hipError_t rmsnorm_fwd(const void* x, const void* g, int dtype, int64_t T, int64_t D, float eps,
                       void* y, float* rstd, int32_t* dflags, hipStream_t s) {
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  int64_t per = cdiv(D, 64 * E);
  int V = 1;
  while (V < per) V *= 2;
  const float invD = 1.0f / (float)D;
  // eps is an input like any other: a subnormal eps reads as a signed zero
  uint32_t eb;
  memcpy(&eb, &eps, 4);
  if ((eb & 0x7f800000u) == 0u) eb &= 0x80000000u;
  float e;
  memcpy(&e, &eb, 4);
  dim3 gr((unsigned)cdiv(T, 4)), b(256);
#define BRQ_F(TT, VV)                                                                            \
  hipLaunchKernelGGL((k_rms_fwd<TT, VV>), gr, b, 0, s, (const TT*)x, (const TT*)g, T, D, invD, \
                     e, (TT*)y, rstd, dflags)
  if (dtype == BRQ_BF16) {
    switch (V) {
      case 1: BRQ_F(uint16_t, 1); break;
      case 2: BRQ_F(uint16_t, 2); break;
      case 4: BRQ_F(uint16_t, 4); break;
      case 8: BRQ_F(uint16_t, 8); break;
      case 16: BRQ_F(uint16_t, 16); break;
      default: BRQ_F(uint16_t, 32); break;
    }
  } else {
    switch (V) {
      case 1: BRQ_F(float, 1); break;
      case 2: BRQ_F(float, 2); break;
      case 4: BRQ_F(float, 4); break;
      case 8: BRQ_F(float, 8); break;
      case 16: BRQ_F(float, 16); break;
      case 32: BRQ_F(float, 32); break;
      default: BRQ_F(float, 64); break;
    }
  }
#undef BRQ_F
  return hipGetLastError();
}

// ---- backward: one work-group (4 waves) per R rows ---------------------------
// Thread t owns vector v's elements [(256 v + t) E, + E) of every row.
//
// The rows' x and dy go from global memory straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the instruction's LDS
// base + 16 l, so wave w's load of vector v fills thread (256 v + 64 w + l)'s
// slot) through kRmsStages stages, issued kRmsStages - 1 rows ahead: each
// work-group keeps three rows in flight without holding them in registers.
// Per row: wait until this wave's loads of the row have landed.  Vector
// memory operations (loads and stores) complete in issue order, so the wait
// allows exactly the operations this wave issued after those loads to stay
// in flight: the later rows' loads and the dx stores of the rows between.
// A store is counted only where the wave certainly issued it (a row inside
// T, a vector with at least one lane inside D): a count that is too low
// only makes the wait stricter.  Then one bare barrier (every wave's part of
// the row is in LDS, every wave has read the previous row's stage and
// written that row's dot partials), finish the previous row (dot, dx, dg
// push), read the row, issue the loads of row + 3 into the freed stage, and
// write the row's dot partials for the next barrier.  Lanes
// past D and rows past T load clamped in-bounds addresses and mask the
// values.
constexpr int kRmsStages = 4;


// ---- unflushed row work of the backward, proved safe from the inputs --------
// A result that is not subnormal is left unchanged by the flush, so a chain
// of operations evaluated without flushes equals the flushed chain whenever
// no intermediate result is subnormal.  For bf16 rows the kernel proves that
// from exponent bounds before evaluating a wave's elements unflushed.  With
// biased exponents Ex, Edy, Eg of the smallest nonzero x, dy, g of a lane
// (after DAZ) and Er of rstd, every rounded product is at least the power of
// two of its operands' bounds (rounding is monotone), so
//   x^ = x rstd       >= 2^(Ex + Er - 254)
//   d  = dy g         >= 2^(Edy + Eg - 254)
//   d x^              >= 2^(Edy + Eg + Ex + Er - 508)
//   dy x^             >= 2^(Edy + Ex + Er - 381)
//   x^ mu             >= 2^(Ex + Er + Emu - 381)
// (or exactly zero).  A value of at least 2^-103 is a multiple of 2^-126,
// and sums and differences of such multiples are multiples of 2^-126 again
// (exact below 2^-102, rounded to a grid of at least 2^-126 above), so they
// are zero or normal.  The conditions therefore are: x^ normal
// (Ex + Er >= 128), d, d x^, dy x^ and x^ mu at least 2^-103
// (Edy + Eg >= 151, Edy + Eg + Ex + Er >= 405, Edy + Ex + Er >= 278,
// Ex + Er + Emu >= 278); then the dot tree, d - x^ mu and the dg stack never
// see a subnormal.  The last product dx = rstd (d - x^ mu) can still be
// subnormal: it is checked (one v_cmp_class per value) and flushed when any
// is.  A wave where a condition fails takes the flushed form.

// Front of one row's work on a lane's E elements: x^ = x rstd, d = dy g,
// the dot leaves d x^ and the dg leaves dy x^ (-0 where the lane's vector
// is padding), and the wave's node of the dot's tree.
template <bool kFast, int E>
__device__ __forceinline__ float rms_bwd_front(const float* xv, const float* dv, const float* gv,
                                               float rs, bool live, float* xh, float* d,
                                               float* leaf) {
  auto mul = [](float a, float b) { return kFast ? a * b : fmul(a, b); };
  auto add = [](float a, float b) { return kFast ? a + b : fadd(a, b); };
  float p[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    xh[e] = mul(xv[e], rs);
    d[e] = mul(dv[e], gv[e]);
    // padding (past D or past T) is -0: exact identity for signed sums
    const float pe = mul(d[e], xh[e]), le = mul(dv[e], xh[e]);
    p[e] = live ? pe : -0.0f;
    leaf[e] = live ? le : -0.0f;
  }
#pragma unroll
  for (int w = E; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) p[i] = add(p[2 * i], p[2 * i + 1]);
  float n = p[0];
  n = add(n, dpp_xor1(n));
  n = add(n, dpp_xor2(n));
  n = add(n, dpp_half_mirror(n));
  n = add(n, dpp_mirror(n));
  LanePair pr = lanes_16(n);
  n = add(pr.lo, pr.hi);
  pr = lanes_32(n);
  n = add(pr.lo, pr.hi);
  return n;
}

template <typename T, int V, int LOGR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(V == 1 ? 4 : 2))) void k_rms_bwd(const T* __restrict__ x, const T* __restrict__ g,
                                                 const float* __restrict__ rstd,
                                                 const T* __restrict__ dy, int64_t Tn, int64_t D,
                                                 float invD, T* __restrict__ dx,
                                                 float* __restrict__ dg_part) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int R = 1 << LOGR;
  constexpr int NE = V * E;
  constexpr int S = kRmsStages;
  constexpr int ROWB = 2 * V * 256 * 16;  // one staged row: x vectors, then dy vectors
  static_assert(R <= 64, "rstd of the block's rows: one per lane");
  // one LDS object: the compiler then does not make the stage reads wait
  // for every direct-to-LDS load in flight
  __shared__ __attribute__((aligned(1024))) uint8_t stage[S * ROWB + 2 * V * 4 * 4];
  float(*red)[V][4] = reinterpret_cast<float(*)[V][4]>(stage + S * ROWB);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * R;

  float gv[NE];
  bool colok[V];
  int64_t coff[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 256 + t) * E;
    colok[v] = c0 < D;
    coff[v] = colok[v] ? c0 : 0;
    if (colok[v]) Elem<T>::unpack(ld16(g + c0), gv + v * E);
    else
#pragma unroll
      for (int e = 0; e < E; ++e) gv[v * E + e] = 0.0f;
  }
  // lane l holds rstd of the block's row l (rows past T: 0)
  const float rs_lane = (lane < R && r0 + lane < Tn) ? flush(rstd[r0 + lane]) : 0.0f;
  float stk[LOGR + 1][NE];
  // biased exponent of the lane's smallest nonzero g per vector (bf16)
  int eg[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    int m = 512;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (gv[v * E + e] != 0.0f && f32_exp(gv[v * E + e]) < m) m = f32_exp(gv[v * E + e]);
    eg[v] = m;
  }
  // sfast: every row pushed on the dg stack so far took the unflushed form
  bool sfast = E == 8;
  // dx store instructions this wave issues per row inside T
  int nst = 0;
#pragma unroll
  for (int v = 0; v < V; ++v) nst += __ballot(colok[v]) != 0 ? 1 : 0;

  auto issue = [&](int rr) {
    int64_t row = r0 + rr;
    row = row < Tn ? row : Tn - 1;
    uint8_t* st = stage + (rr % S) * ROWB;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      __builtin_amdgcn_global_load_lds(
          (const void*)(x + row * D + coff[v]),
          (__attribute__((address_space(3))) void*)(st + (v * 256 + wave * 64) * 16), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const void*)(dy + row * D + coff[v]),
          (__attribute__((address_space(3))) void*)(st + ((V + v) * 256 + wave * 64) * 16), 16,
          0, 0);
    }
  };
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < R) issue(s);

  // bf16 rows take the unflushed form where the exponent bounds allow
  constexpr bool kSpec = E == 8;
  // the row in flight between its front (before a barrier) and its back
  // (after it): x^, d, dg leaves, rstd, exponent bounds
  float xh[NE], d[NE], leaf[NE];
  int exv[V];
  float rs = 0.0f;
  bool lfast = true;  // every vector of the row took the unflushed form

  // One barrier per row: iteration rr waits for row rr's loads, then (after
  // the barrier, which also publishes row rr - 1's dot partials) finishes
  // row rr - 1 and starts row rr, whose partials the next barrier publishes.
#pragma unroll 1
  for (int rr = 0; rr <= R; ++rr) {
    if (rr < R) {
      const int later = (R - 1 - rr) < (S - 2) ? (R - 1 - rr) : (S - 2);
      // rows whose dx stores were issued after this row's loads: those of
      // [rr - S + 1, rr - 2] inside T
      const int w0 = rr - S + 1 > 0 ? rr - S + 1 : 0;
      const int64_t w1 = r0 + rr - 2 < Tn - 1 ? r0 + rr - 2 : Tn - 1;  // last row inside T
      const int nrows = (int)(w1 - (r0 + w0) + 1) > 0 ? (int)(w1 - (r0 + w0) + 1) : 0;
      wait_vmcnt_upto<3 * V * (S - 2)>(2 * V * later + nst * nrows);
    }
    // this wave's dot partials of row rr - 1 are in LDS; a bare barrier (a
    // fenced one would also wait for the rows in flight)
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    if (rr > 0) {
      // back of row pr = rr - 1 (its dot partials are in red[pr & 1]): dx,
      // then the binary-carry push of its dg leaves
      const int pr = rr - 1;
      const int64_t row = r0 + pr;
      const bool rowok = row < Tn;  // uniform across the work-group
      float n4[V];
#pragma unroll
      for (int v = 0; v < V; ++v)
        n4[v] = fadd(fadd(red[pr & 1][v][0], red[pr & 1][v][1]),
                     fadd(red[pr & 1][v][2], red[pr & 1][v][3]));
      const float dot = reg_tree<true, V>(n4);
      const float mu = fmul(dot, invD);
      // exponent bound of mu (a zero mu makes x^ mu an exact zero)
      const int emu = mu == 0.0f ? 512 : f32_exp(mu);
      const int er = f32_exp(rs);
      if (rowok) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int64_t c0 = (int64_t)(v * 256 + t) * E;
          if (!colok[v]) continue;
          const int k0 = v * E;
          float o[E];
          bool fast = false;
          if constexpr (kSpec) fast = lfast && __ballot(exv[v] + er + emu < 278) == 0;
          if (fast) {
            uint64_t bad = 0;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              o[e] = rs * (d[k0 + e] - xh[k0 + e] * mu);
              bad |= sub_mask(o[e]);
            }
            if (bad)
#pragma unroll
              for (int e = 0; e < E; ++e) o[e] = flush(o[e]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
              o[e] = fmul(rs, fsub(d[k0 + e], fmul(xh[k0 + e], mu)));
          }
          st16(dx + row * D + c0, pack_out<T>(o));
        }
      }
      // every dg leaf pushed so far is zero or at least 2^-103 while sfast
      // holds: the stack's sums need no flush
      sfast = __builtin_amdgcn_readfirstlane(sfast && lfast);
      // row pr merges with the pending nodes of the levels where pr has a 1
      // bit (lowest first)
      bool carry = true;
#pragma unroll
      for (int l = 0; l <= LOGR; ++l) {
        if (carry) {
          if ((pr >> l) & 1) {
            if (sfast) {
#pragma unroll
              for (int k = 0; k < NE; ++k) leaf[k] = stk[l][k] + leaf[k];
            } else {
#pragma unroll
              for (int k = 0; k < NE; ++k) leaf[k] = fadd(stk[l][k], leaf[k]);
            }
          } else {
#pragma unroll
            for (int k = 0; k < NE; ++k) stk[l][k] = leaf[k];
            carry = false;
          }
        }
      }
    }
    if (rr == R) break;

    const int64_t row = r0 + rr;
    const bool rowok = row < Tn;  // uniform across the work-group
    const uint8_t* st = stage + (rr % S) * ROWB;
    u32x4 xc[V], dc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      xc[v] = *reinterpret_cast<const u32x4*>(st + (v * 256 + t) * 16);
      dc[v] = *reinterpret_cast<const u32x4*>(st + ((V + v) * 256 + t) * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (rr + S - 1 < R) issue(rr + S - 1);
    __builtin_amdgcn_sched_barrier(0);
    rs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rs_lane), rr));
    lfast = true;
    const int er = f32_exp(rs);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float xv[E], dv[E];
      const bool live = rowok && colok[v];
      const int k0 = v * E;
      float nd;
      if constexpr (kSpec) {
        const int ex = widen_bf16x8_daz(xc[v], xv);
        const int ed = widen_bf16x8_daz(dc[v], dv);
        exv[v] = ex;
        const bool ok = ex + er >= 128 && ed + eg[v] >= 151 && ed + eg[v] + ex + er >= 405 &&
                        ed + ex + er >= 278;
        const bool fast = __ballot(!ok) == 0;  // wave-uniform
        lfast = lfast && fast;
        if (fast) nd = rms_bwd_front<true, E>(xv, dv, gv + k0, rs, live, xh + k0, d + k0, leaf + k0);
        else nd = rms_bwd_front<false, E>(xv, dv, gv + k0, rs, live, xh + k0, d + k0, leaf + k0);
      } else {
        Elem<T>::unpack(xc[v], xv);
        Elem<T>::unpack(dc[v], dv);
        nd = rms_bwd_front<false, E>(xv, dv, gv + k0, rs, live, xh + k0, d + k0, leaf + k0);
      }
      if (lane == 0) red[rr & 1][v][wave] = nd;
    }
  }
  // R is a power of two: the block's node sits at level LOGR.
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 256 + t) * E;
    if (!colok[v]) continue;
#pragma unroll
    for (int e = 0; e < E; e += 4)
      st16(dg_part + (int64_t)blockIdx.x * D + c0 + e,
           u32x4{__float_as_uint(stk[LOGR][v * E + e]), __float_as_uint(stk[LOGR][v * E + e + 1]),
                 __float_as_uint(stk[LOGR][v * E + e + 2]),
                 __float_as_uint(stk[LOGR][v * E + e + 3])});
  }
}

// Next tree levels over the per-block nodes: in [P][D] holds node(l, p) of
// every column for p < P; a lane owns 4 columns of one aligned group of
// 32 nodes and folds them with the same binary-carry stack (nodes past P are
// -0, the exact identity), giving node(l + 5, q) in out [ceil(P/32)][D].
constexpr int kFoldLog = 5;
__global__ __launch_bounds__(256) void k_dg_fold(const float* __restrict__ in, int64_t P, int64_t D,
                                                 int64_t col_blocks, float* __restrict__ out) {
  const int64_t q = (int64_t)blockIdx.x / col_blocks;
  const int64_t c = (((int64_t)blockIdx.x % col_blocks) * 256 + threadIdx.x) * 4;
  if (c >= D) return;
  float stk[kFoldLog + 1][4];
  // every load of the group first (one round trip), then the stack
  float4 v4[1 << kFoldLog];
#pragma unroll
  for (int i = 0; i < (1 << kFoldLog); ++i) {
    const int64_t p = q * (1 << kFoldLog) + i;
    v4[i] = p < P ? *reinterpret_cast<const float4*>(in + p * D + c)
                  : make_float4(-0.0f, -0.0f, -0.0f, -0.0f);
  }
#pragma unroll
  for (int i = 0; i < (1 << kFoldLog); ++i) {
    float val[4] = {v4[i].x, v4[i].y, v4[i].z, v4[i].w};
    bool carry = true;
#pragma unroll
    for (int l = 0; l <= kFoldLog; ++l) {
      if (carry) {
        if ((i >> l) & 1) {
#pragma unroll
          for (int k = 0; k < 4; ++k) val[k] = fadd(stk[l][k], val[k]);
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) stk[l][k] = val[k];
          carry = false;
        }
      }
    }
  }
  *reinterpret_cast<float4*>(out + q * D + c) =
      make_float4(stk[kFoldLog][0], stk[kFoldLog][1], stk[kFoldLog][2], stk[kFoldLog][3]);
}

// dg of an empty token range: the tree over no leaves is +0.
__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

int rmsnorm_bwd_rows(int64_t D, int dtype, const brq_tune* t) {
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  int64_t per = cdiv(D, 256 * E);
  int V = 1;
  while (V < per) V *= 2;
  // default: 8 rows per block for one vector per lane (the 2048-wide bf16
  // rows measured fastest there, 4% ahead of 32 with its one fold level
  // fewer), else 32 / V
  int R = (t && t->rows_per_block) ? t->rows_per_block : (V == 1 ? 8 : 32 / V);
  int cap = 32 / V;
  if (R > cap) R = cap;
  int r = 1;
  while (r * 2 <= R) r *= 2;
  return r;
}

size_t rmsnorm_bwd_ws(int64_t T, int64_t D, int dtype, const brq_tune* t) {
  int R = rmsnorm_bwd_rows(D, dtype, t);
  const int64_t P = cdiv(T > 0 ? T : 1, R);
  return align256((size_t)P * (size_t)D * sizeof(float)) +
         align256((size_t)cdiv(P, 1 << kFoldLog) * (size_t)D * sizeof(float));
}

template <typename TT, int VV>
static void launch_bwd(int R, dim3 gr, hipStream_t s, const void* x, const void* g,
                       const float* rstd, const void* dy, int64_t T, int64_t D, float invD,
                       void* dx, float* part) {
  dim3 b(256);
#define BRQ_B(LR)                                                                        \
  hipLaunchKernelGGL((k_rms_bwd<TT, VV, LR>), gr, b, 0, s, (const TT*)x, (const TT*)g, rstd, \
                     (const TT*)dy, T, D, invD, (TT*)dx, part)
  switch (R) {
    case 1: BRQ_B(0); break;
    case 2: BRQ_B(1); break;
    case 4: BRQ_B(2); break;
    case 8: BRQ_B(3); break;
    case 16: BRQ_B(4); break;
    default: BRQ_B(5); break;
  }
#undef BRQ_B
}

hipError_t rmsnorm_bwd(const void* x, const void* g, const float* rstd, const void* dy, int dtype,
                       int64_t T, int64_t D, void* dx, float* dg, void* ws, const brq_tune* t,
                       hipStream_t s) {
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  int64_t per = cdiv(D, 256 * E);
  int V = 1;
  while (V < per) V *= 2;
  const int R = rmsnorm_bwd_rows(D, dtype, t);
  const int64_t P = cdiv(T, R);
  const float invD = 1.0f / (float)D;
  float* part = (float*)ws;
  dim3 gr((unsigned)(P > 0 ? P : 0));
  if (P > 0) {
    if (dtype == BRQ_BF16) {
      if (V == 1) launch_bwd<uint16_t, 1>(R, gr, s, x, g, rstd, dy, T, D, invD, dx, part);
      else launch_bwd<uint16_t, 2>(R, gr, s, x, g, rstd, dy, T, D, invD, dx, part);
    } else {
      if (V == 1) launch_bwd<float, 1>(R, gr, s, x, g, rstd, dy, T, D, invD, dx, part);
      else launch_bwd<float, 2>(R, gr, s, x, g, rstd, dy, T, D, invD, dx, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (P == 0) {
    hipLaunchKernelGGL(k_zero_f32, dim3((unsigned)cdiv(D, 256)), dim3(256), 0, s, dg, D);
    return hipGetLastError();
  }
  // fold the per-block nodes 32 at a time until one row remains (at least
  // once, so that the last fold writes dg itself)
  float* bufs[2] = {part, part + align256((size_t)P * (size_t)D * sizeof(float)) / sizeof(float)};
  const float* cur = part;
  int64_t n = P;
  int which = 1;
  const int64_t cb = cdiv(D, 1024);
  do {
    const int64_t nn = cdiv(n, 1 << kFoldLog);
    float* dst = nn == 1 ? dg : bufs[which];
    hipLaunchKernelGGL(k_dg_fold, dim3((unsigned)(nn * cb)), dim3(256), 0, s, cur, n, D, cb, dst);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    cur = dst;
    which ^= 1;
    n = nn;
  } while (n > 1);
  return hipSuccess;
}

// ---- global gradient norm ------------------------------------------------------
// S = the tree sum of squares, norm = fl(sqrt S): computed by the
// reduction's final work-group
hipError_t grad_norm(const float* v, int64_t n, float* sumsq, float* norm, void* ws,
                     int chunk_log2, int32_t* dflags, hipStream_t s) {
  float* sum2 = (float*)ws;
  void* fws = (char*)ws + 256;
  const FlatFin fin{FIN_NORM, 0.0f, nullptr, nullptr, nullptr, sumsq, norm};
  return flat_reduce(v, BRQ_F32, LEAF_SQUARE, nullptr, n, 1, sum2, fws, chunk_log2, dflags, s, 0,
                     &fin);
}

}  // namespace brq
