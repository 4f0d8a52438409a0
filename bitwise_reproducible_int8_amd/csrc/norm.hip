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
  u32x4 raw[V];
  float node[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    raw[v] = c0 < D ? ld16(xr + c0) : u32x4{0, 0, 0, 0};
    float f[E];
    Elem<T>::unpack(raw[v], f);
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = flush_nonneg(f[e] * f[e]);
    node[v] = wave_tree<false>(reg_tree<false, E>(f));
  }
  const float ss = reg_tree<false, V>(node);
  const float ms = fmul(ss, invD);
  const float r = flush(1.0f / flush(__builtin_sqrtf(fadd(ms, eps))));
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    if (c0 >= D) continue;
    float f[E], gv[E], o[E];
    Elem<T>::unpack(raw[v], f);
    Elem<T>::unpack(ld16(g + c0), gv);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = fmul(fmul(f[e], r), gv[e]);
    if (E == 8) {
      st16(y + row * D + c0, pack_out<T>(o));
    } else {
      st16(y + row * D + c0, pack_out<T>(o));
    }
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
  const float e = eps;
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
template <typename T, int V, int LOGR>
__global__ __launch_bounds__(256) void k_rms_bwd(const T* __restrict__ x, const T* __restrict__ g,
                                                 const float* __restrict__ rstd,
                                                 const T* __restrict__ dy, int64_t Tn, int64_t D,
                                                 float invD, T* __restrict__ dx,
                                                 float* __restrict__ dg_part) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int R = 1 << LOGR;
  constexpr int NE = V * E;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * R;
  __shared__ float red[2][V][4];

  float gv[NE];
  bool colok[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 256 + t) * E;
    colok[v] = c0 < D;
    if (colok[v]) Elem<T>::unpack(ld16(g + c0), gv + v * E);
    else
#pragma unroll
      for (int e = 0; e < E; ++e) gv[v * E + e] = 0.0f;
  }
  float stk[LOGR + 1][NE];

  // raw 16-byte vectors of the next row: its loads are in flight while the
  // current row is reduced and written
  u32x4 xn[V], dn[V];
  auto fetch = [&](int rr) {
    const int64_t row = r0 + rr;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int64_t c0 = (int64_t)(v * 256 + t) * E;
      const bool ok = rr < R && row < Tn && colok[v];
      xn[v] = ok ? ld16(x + row * D + c0) : u32x4{0, 0, 0, 0};
      dn[v] = ok ? ld16(dy + row * D + c0) : u32x4{0, 0, 0, 0};
    }
  };
  fetch(0);

#pragma unroll 1
  for (int rr = 0; rr < R; ++rr) {
    const int64_t row = r0 + rr;
    const bool rowok = row < Tn;  // uniform across the work-group
    u32x4 xc[V], dc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) { xc[v] = xn[v]; dc[v] = dn[v]; }
    fetch(rr + 1);
    float xh[NE], d[NE], leaf[NE];
    const float rs = rowok ? flush(rstd[row]) : 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      float xv[E], dv[E];
      Elem<T>::unpack(xc[v], xv);
      Elem<T>::unpack(dc[v], dv);
      float p[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int k = v * E + e;
        xh[k] = fmul(xv[e], rs);
        d[k] = fmul(dv[e], gv[k]);
        // padding (past D or past T) is -0: exact identity for signed sums
        p[e] = (rowok && colok[v]) ? fmul(d[k], xh[k]) : -0.0f;
        leaf[k] = (rowok && colok[v]) ? fmul(dv[e], xh[k]) : -0.0f;
      }
      float nd = wave_tree<true>(reg_tree<true, E>(p));
      if (lane == 0) red[rr & 1][v][wave] = nd;
    }
    __syncthreads();
    float n4[V];
#pragma unroll
    for (int v = 0; v < V; ++v)
      n4[v] = fadd(fadd(red[rr & 1][v][0], red[rr & 1][v][1]),
                   fadd(red[rr & 1][v][2], red[rr & 1][v][3]));
    const float dot = reg_tree<true, V>(n4);
    const float mu = fmul(dot, invD);
    if (rowok) {
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int64_t c0 = (int64_t)(v * 256 + t) * E;
        if (!colok[v]) continue;
        float o[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int k = v * E + e;
          o[e] = fmul(rs, fsub(d[k], fmul(xh[k], mu)));
        }
        st16(dx + row * D + c0, pack_out<T>(o));
      }
    }
    // binary-carry push of this row's dg leaves: row rr merges with the
    // pending nodes of the levels where rr has a 1 bit (lowest first)
    bool carry = true;
#pragma unroll
    for (int l = 0; l <= LOGR; ++l) {
      if (carry) {
        if ((rr >> l) & 1) {
#pragma unroll
          for (int k = 0; k < NE; ++k) leaf[k] = fadd(stk[l][k], leaf[k]);
        } else {
#pragma unroll
          for (int k = 0; k < NE; ++k) stk[l][k] = leaf[k];
          carry = false;
        }
      }
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
  int R = (t && t->rows_per_block) ? t->rows_per_block : 32 / V;
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
__global__ void k_gn_finalize(const float* sum_max, float* sumsq, float* norm) {
  const float ss = sum_max[0];
  sumsq[0] = ss;
  norm[0] = flush(__builtin_sqrtf(ss));
}

hipError_t grad_norm(const float* v, int64_t n, float* sumsq, float* norm, void* ws,
                     int chunk_log2, int32_t* dflags, hipStream_t s) {
  float* sum2 = (float*)ws;
  void* fws = (char*)ws + 256;
  hipError_t e = flat_reduce(v, BRQ_F32, LEAF_SQUARE, nullptr, n, 1, sum2, fws, chunk_log2, dflags, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gn_finalize, dim3(1), dim3(1), 0, s, sum2, sumsq, norm);
  return hipGetLastError();
}

}  // namespace brq
