// quant.hip -- LSQ int8 quantisation on gfx950 (Open-1B report §3.1 "int8
// quantization-aware training", §4.2 "Implementation notes", §3.2 "int8
// computation"): step size s = 2*mean(|v|)/sqrt(127) recomputed from the
// tensor, q = clamp(rint(v / s), -127, 127) with the divide done as a
// multiply by fl(1/s) (App. A.3).
//
// Per-tensor groups take two passes over the input: the statistic (a
// canonical-tree sum of |v| plus max|v|) and then the codes.  The tree is
// cut into aligned power-of-two chunks, one per work-group: every chunk is a
// complete subtree of the whole-tensor tree, so summing the chunk sums with
// the same pairwise rule gives exactly the whole-tensor tree, whatever the
// chunk size, wave size or grid size.  Lanes beyond the end contribute +0,
// an exact identity for these non-negative leaves (it equals the "unpaired
// node moves up" rule).
//
// Per-row groups (weights, one step size per output channel) fit in one
// wave: one read, one write.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

// --------------------------------------------------------------------------
// flat tree, pass 1: one aligned chunk of C = 4 waves * 64 lanes * V vectors
// * E elements per work-group.  Vector v of lane l covers elements
// [wave_base + (64 v + l) E, + E): each wave-wide vector load is one
// contiguous 64*16-byte run, and the 64 lanes' subtrees pair up through the
// butterfly into node(log2(64E), .) of that run.
// --------------------------------------------------------------------------
template <typename T, int LEAF, int B = 0>
__device__ __forceinline__ void leaves_of(const T* x, const float* cm, int64_t n,
                                          int64_t cols, int64_t idx0, float* f) {
  constexpr int E = Elem<T>::kPerVec;
  if (B > 0) {
    // |rows rotation of (x * cm)|: n % B == 0, so a vector is wholly in
    // range or wholly past the end (zeros).  Evaluated without flushes
    // first; any subnormal value in the wave redoes it with them.  Every
    // lane of the wave reaches the butterflies and the test.
    const u32x4 raw = idx0 < n ? ld16(x + idx0) : u32x4{0, 0, 0, 0};
    const int64_t col = col_of(idx0, cols);
    float m[E];
    uint64_t bad = 0;
    widen_raw<T>(raw, f, bad);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      m[e] = cm[col + e];
      bad |= sub_mask(m[e]);
      f[e] = f[e] * m[e];
      bad |= sub_mask(f[e]);
    }
    wht_block_fast<E, B>(f, threadIdx.x & 63, bad);
    if (bad) {
      Elem<T>::unpack(raw, f);
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] = fmul(f[e], flush(m[e]));
      wht_block<E, B>(f, threadIdx.x & 63);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = fabs_bits(f[e]);
    return;
  }
  if (idx0 + E <= n) {
    Elem<T>::unpack(ld16(x + idx0), f);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = (idx0 + e < n) ? Elem<T>::load1(x, idx0 + e) : 0.0f;
  }
  if (LEAF == LEAF_ABS_COLMUL) {
    int64_t col = idx0 % cols;  // cols % E == 0: the vector sits in one row
#pragma unroll
    for (int e = 0; e < E; ++e) f[e] = fmul(f[e], flush(cm[col + e]));
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (LEAF == LEAF_SQUARE) f[e] = flush_nonneg(f[e] * f[e]);
    else if (LEAF != LEAF_RAW) f[e] = fabs_bits(f[e]);
  }
}

// Raw fp32 leaves idx0 .. idx0 + 3 of an array stored tile by tile
// (TileMap); leaves past n are 0.  Two leaves (row, c), (row, c + 1) with c
// even sit side by side, so when nb is an even power of two (idx0 % 4 == 0,
// the four leaves in one row) two 8-byte loads fetch them.
__device__ __forceinline__ int64_t tile_index(int64_t i, const TileMap& m) {
  int64_t row, c;
  if (m.lognb >= 0) {
    row = i >> m.lognb;
    c = i & (m.nb - 1);
  } else {
    row = i / m.nb;
    c = i - row * m.nb;
  }
  return (((row >> 7) * m.gx + (c >> 1)) << 8) + ((row & 127) << 1) + (c & 1);
}
__device__ __forceinline__ void leaves_tiled(const float* x, int64_t n, const TileMap& m,
                                             int64_t idx0, float* f) {
  if (m.lognb >= 2 && idx0 + 4 <= n) {
    const float2 a = *reinterpret_cast<const float2*>(x + tile_index(idx0, m));
    const float2 b = *reinterpret_cast<const float2*>(x + tile_index(idx0 + 2, m));
    f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = idx0 + e < n ? x[tile_index(idx0 + e, m)] : 0.0f;
  }
}

template <typename T, int LEAF, int V, int B = 0, bool TILED = false>
__device__ __forceinline__ void flat_leaves_body(const T* __restrict__ x,
                                                 const float* __restrict__ cm, int64_t n,
                                                 int64_t cols, float* __restrict__ psum,
                                                 float* __restrict__ pmax,
                                                 const TileMap tm = TileMap{0, 0, -1}) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int64_t WAVE_SPAN = int64_t(64) * E * V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t base = (int64_t)blockIdx.x * 4 * WAVE_SPAN + wave * WAVE_SPAN;
  float node[V];
  float mx = 0.0f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float f[E];
    if constexpr (TILED)
      leaves_tiled(reinterpret_cast<const float*>(x), n, tm, base + (int64_t)(v * 64 + lane) * E,
                   f);
    else
      leaves_of<T, LEAF, B>(x, cm, n, cols, base + (int64_t)(v * 64 + lane) * E, f);
#pragma unroll
    for (int e = 0; e < E; ++e) mx = fmaxf(mx, f[e]);
    node[v] = wave_tree<false>(reg_tree<false, E>(f));
  }
  float w = reg_tree<false, V>(node);
  mx = wave_max(mx);
  __shared__ float sw[4], sm[4];
  if (lane == 0) { sw[wave] = w; sm[wave] = mx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    psum[blockIdx.x] = (sw[0] + sw[1]) + (sw[2] + sw[3]);
    pmax[blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  }
}

template <typename T, int LEAF, int V>
__global__ __launch_bounds__(256) void k_flat_leaves(const T* __restrict__ x,
                                                     const float* __restrict__ cm,
                                                     int64_t n, int64_t cols,
                                                     float* __restrict__ psum,
                                                     float* __restrict__ pmax) {
  flat_leaves_body<T, LEAF, V>(x, cm, n, cols, psum, pmax);
}

// The leaves |rows rotation of (x * cm)| in blocks of B along each row
// (B <= 64 E, so every block sits in consecutive lanes of one wave).
template <typename T, int V, int B>
__global__ __launch_bounds__(256) void k_flat_leaves_wht(const T* __restrict__ x,
                                                         const float* __restrict__ cm,
                                                         int64_t n, int64_t cols,
                                                         float* __restrict__ psum,
                                                         float* __restrict__ pmax) {
  flat_leaves_body<T, LEAF_ABS_COLMUL, V, B>(x, cm, n, cols, psum, pmax);
}

// Two independent raw-leaf reductions of equal length in one launch:
// blockIdx.y selects the array.
struct FlatPair {
  const float* x[2];
  float* ps[2];
  float* pm[2];
};
template <int V>
__global__ __launch_bounds__(256) void k_flat_leaves_pair(FlatPair a, int64_t n) {
  const int y = blockIdx.y;
  flat_leaves_body<float, LEAF_RAW, V>(a.x[y], nullptr, n, 1, a.ps[y], a.pm[y]);
}
// the same over two arrays stored tile by tile
template <int V>
__global__ __launch_bounds__(256) void k_flat_leaves_pair_tiled(FlatPair a, int64_t n, TileMap tm) {
  const int y = blockIdx.y;
  flat_leaves_body<float, LEAF_RAW, V, 0, true>(a.x[y], nullptr, n, 1, a.ps[y], a.pm[y], tm);
}

// Final level: up to 32768 partials in one work-group of 1024 lanes, each
// lane an aligned run of 32.  Writes out[0] = sum, out[1] = max.
__device__ __forceinline__ void flat_final_body(const float* __restrict__ psum,
                                                const float* __restrict__ pmax, int64_t P,
                                                float* out, int32_t* flags, float* s_out = nullptr,
                                                float* m_out = nullptr) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float a[32];
  float mx = 0.0f;
  const int64_t j0 = (int64_t)t * 32;
  if (j0 + 32 <= P) {
    // both arrays start 16-byte aligned: eight 16-byte loads each
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(psum + j0 + 4 * i);
      const float4 m = *reinterpret_cast<const float4*>(pmax + j0 + 4 * i);
      a[4 * i] = v.x; a[4 * i + 1] = v.y; a[4 * i + 2] = v.z; a[4 * i + 3] = v.w;
      mx = fmaxf(fmaxf(mx, fmaxf(m.x, m.y)), fmaxf(m.z, m.w));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int64_t j = j0 + i;
      a[i] = j < P ? psum[j] : 0.0f;
      mx = fmaxf(mx, j < P ? pmax[j] : 0.0f);
    }
  }
  float w = wave_tree<false>(reg_tree<false, 32>(a));
  mx = wave_max(mx);
  __shared__ float sw[16], sm[16];
  if (lane == 0) { sw[wave] = w; sm[wave] = mx; }
  __syncthreads();
  if (t == 0) {
    float b[16], m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) { b[i] = sw[i]; m = fmaxf(m, sm[i]); }
    float s = reg_tree<false, 16>(b);
    out[0] = s;
    out[1] = m;
    if (!__builtin_isfinite(s)) set_flag(flags, BRQ_FLAG_NONFINITE);
    if (s_out) *s_out = s;
    if (m_out) *m_out = m;
  }
}

// LSQ step size and reciprocal from a tree sum S (the operations of
// k_lsq_finalize): m = fl(S * inv_n), s = fl(m * K2), r = fl(1/s).
__device__ __forceinline__ void lsq_step(float S, float inv_n, float& sc, float& r) {
  sc = fmul(fmul(S, inv_n), lsq_k2());
  r = (sc == 0.0f) ? 0.0f : fl_div(1.0f, sc);
}

__global__ __launch_bounds__(1024) void k_flat_final(const float* __restrict__ psum,
                                                     const float* __restrict__ pmax,
                                                     int64_t P, float* out, int32_t* flags,
                                                     FlatFin fin) {
  float S = 0.0f, M = 0.0f;
  flat_final_body(psum, pmax, P, out, flags, &S, &M);
  if (threadIdx.x != 0) return;
  if (fin.kind == FIN_LSQ) {
    float sc, r;
    lsq_step(S, fin.inv_n, sc, r);
    fin.sr[0] = sc;
    fin.sr[1] = r;
    if (fin.scale) fin.scale[0] = sc;
    if (fin.amax) fin.amax[0] = M;
  } else if (fin.kind == FIN_NORM) {
    fin.sumsq[0] = S;
    fin.norm[0] = fl_sqrt(S);
  }
}

// blockIdx.x selects the array of the pair
__global__ __launch_bounds__(1024) void k_flat_final_pair(FlatPair a, int64_t P, float* out0,
                                                          float* out1, int32_t* flags,
                                                          PairFin fin) {
  const int y = blockIdx.x;
  float S = 0.0f;
  flat_final_body(a.ps[y], a.pm[y], P, y ? out1 : out0, flags, &S);
  if (!fin.on) return;
  float m = 0.0f;
  if (y == 0) {
    // order-free max of the work-group maxima
    for (int64_t i = threadIdx.x; i < fin.nb; i += 1024) m = fmaxf(m, fin.bmax[i]);
    m = wave_max(m);
    __shared__ float wm[16];
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, wm[i]);
  }
  if (threadIdx.x != 0) return;
  float sc, r;
  lsq_step(S, fin.inv_n, sc, r);
  fin.sr4[2 * y] = sc;
  fin.sr4[2 * y + 1] = r;
  if (y == 0) {
    if (fin.s0) fin.s0[0] = sc;
    if (fin.amax0) fin.amax0[0] = m;
  } else if (fin.s1) {
    fin.s1[0] = sc;
  }
}

int flat_chunk_log2(const brq_tune* t) {
  int c = (t && t->chunk_log2) ? t->chunk_log2 : 13;
  return c < 10 ? 10 : (c > 16 ? 16 : c);
}

static int vectors_for(int chunk_log2, int E) {
  int v = (int)((1ll << chunk_log2) / (256 * E));
  return v < 1 ? 1 : (v > 16 ? 16 : v);
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of partials after each pass; the last level holds <= 32768.
static int levels_of(int64_t n, int64_t C0, int64_t C, int64_t* P, int maxlev) {
  int L = 0;
  P[L++] = cdiv(n > 0 ? n : 1, C0);
  while (P[L - 1] > 32768 && L < maxlev) { P[L] = cdiv(P[L - 1], C); ++L; }
  return L;
}

// Each level holds P sums, then P maxima from the next 16-byte boundary:
// 4 round4(P) + 4 P <= align256(8 P) for every P, so the level's share of
// the workspace is unchanged.
size_t flat_reduce_ws(int64_t n, int chunk_log2) {
  int64_t P[16];
  int64_t C0 = int64_t(256) * 8 * vectors_for(chunk_log2, 8);  // conservative (bf16 chunk)
  int64_t C0f = int64_t(256) * 4 * vectors_for(chunk_log2, 4);
  if (C0f < C0) C0 = C0f;
  int L = levels_of(n, C0, int64_t(256) * 4 * 16, P, 16);
  size_t b = 0;
  for (int i = 0; i < L; ++i) b += align256(2 * sizeof(float) * (size_t)P[i]);
  return b + 256;
}

template <typename T, int LEAF>
static hipError_t launch_leaves(const T* x, const float* cm, int64_t n, int64_t cols, int V,
                                int64_t P, float* ps, float* pm, hipStream_t s) {
  dim3 g((unsigned)P), b(256);
  switch (V) {
    case 1: hipLaunchKernelGGL((k_flat_leaves<T, LEAF, 1>), g, b, 0, s, x, cm, n, cols, ps, pm); break;
    case 2: hipLaunchKernelGGL((k_flat_leaves<T, LEAF, 2>), g, b, 0, s, x, cm, n, cols, ps, pm); break;
    case 4: hipLaunchKernelGGL((k_flat_leaves<T, LEAF, 4>), g, b, 0, s, x, cm, n, cols, ps, pm); break;
    case 8: hipLaunchKernelGGL((k_flat_leaves<T, LEAF, 8>), g, b, 0, s, x, cm, n, cols, ps, pm); break;
    default: hipLaunchKernelGGL((k_flat_leaves<T, LEAF, 16>), g, b, 0, s, x, cm, n, cols, ps, pm); break;
  }
  return hipGetLastError();
}

// Max partials of a level: one work-group per 16384 entries of the level
// below, matching the raw-sum pass, so both arrays have the same length.
// (max is order-free: any grouping is exact.)
__device__ __forceinline__ void max_partials_body(const float* __restrict__ pm, int64_t P,
                                                  float* __restrict__ out) {
  const int64_t i0 = (int64_t)blockIdx.x * 16384;
  float m = 0.0f;
  for (int i = threadIdx.x; i < 16384; i += 256) {
    int64_t j = i0 + i;
    if (j < P) m = fmaxf(m, pm[j]);
  }
  m = wave_max(m);
  __shared__ float sm[4];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
}

__global__ __launch_bounds__(256) void k_max_partials(const float* __restrict__ pm, int64_t P,
                                                      float* __restrict__ out) {
  max_partials_body(pm, P, out);
}

// pm_in = the pair's level below, pm_out = this level (blockIdx.y selects)
__global__ __launch_bounds__(256) void k_max_partials_pair(FlatPair below, FlatPair level,
                                                           int64_t P) {
  const int y = blockIdx.y;
  max_partials_body(below.pm[y], P, level.pm[y]);
}

// Level 0 of the rows-rotation leaves: V = vectors_for(13, E) (4 for bf16,
// 8 for fp32; the tree does not depend on the chunk), B a power of two.
template <typename T, int V>
static hipError_t launch_leaves_wht(const T* x, const float* cm, int64_t n, int64_t cols, int B,
                                    int64_t P, float* ps, float* pm, hipStream_t s) {
  dim3 g((unsigned)P), b(256);
#define BRQ_LW(BB) hipLaunchKernelGGL((k_flat_leaves_wht<T, V, BB>), g, b, 0, s, x, cm, n, cols, ps, pm)
  switch (B) {
    case 1: BRQ_LW(1); break;
    case 2: BRQ_LW(2); break;
    case 4: BRQ_LW(4); break;
    case 8: BRQ_LW(8); break;
    case 16: BRQ_LW(16); break;
    case 32: BRQ_LW(32); break;
    case 64: BRQ_LW(64); break;
    default: BRQ_LW(128); break;
  }
#undef BRQ_LW
  return hipGetLastError();
}

hipError_t flat_reduce(const void* x, int dtype, int leaf, const float* col_mul, int64_t n,
                       int64_t cols, float* out2, void* ws, int chunk_log2, int32_t* dflags,
                       hipStream_t s, int wht_block, const FlatFin* fin) {
  if (wht_block > 0) chunk_log2 = 13;
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  const int V = vectors_for(chunk_log2, E);
  const int64_t C0 = int64_t(256) * E * V;
  const int Vr = 16;  // raw partial levels: 16384 leaves per work-group
  int64_t P[16];
  int L = levels_of(n, C0, int64_t(256) * 4 * Vr, P, 16);
  char* w = (char*)ws;
  float* ps[16];
  float* pm[16];
  for (int i = 0; i < L; ++i) {
    ps[i] = (float*)w;
    pm[i] = ps[i] + ((P[i] + 3) & ~int64_t(3));  // 16-byte aligned (fits: see flat_reduce_ws)
    w += align256(2 * sizeof(float) * (size_t)P[i]);
  }
  hipError_t e;
  if (wht_block > 0) {
    if (dtype == BRQ_BF16)
      e = launch_leaves_wht<uint16_t, 4>((const uint16_t*)x, col_mul, n, cols, wht_block, P[0],
                                         ps[0], pm[0], s);
    else
      e = launch_leaves_wht<float, 8>((const float*)x, col_mul, n, cols, wht_block, P[0], ps[0],
                                      pm[0], s);
  } else if (dtype == BRQ_BF16) {
    const uint16_t* xb = (const uint16_t*)x;
    if (leaf == LEAF_ABS) e = launch_leaves<uint16_t, LEAF_ABS>(xb, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
    else if (leaf == LEAF_ABS_COLMUL) e = launch_leaves<uint16_t, LEAF_ABS_COLMUL>(xb, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
    else e = launch_leaves<uint16_t, LEAF_SQUARE>(xb, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
  } else {
    const float* xf = (const float*)x;
    if (leaf == LEAF_ABS) e = launch_leaves<float, LEAF_ABS>(xf, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
    else if (leaf == LEAF_ABS_COLMUL) e = launch_leaves<float, LEAF_ABS_COLMUL>(xf, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
    else if (leaf == LEAF_SQUARE) e = launch_leaves<float, LEAF_SQUARE>(xf, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
    else e = launch_leaves<float, LEAF_RAW>(xf, col_mul, n, cols, V, P[0], ps[0], pm[0], s);
  }
  if (e != hipSuccess) return e;
  for (int i = 1; i < L; ++i) {
    e = launch_leaves<float, LEAF_RAW>(ps[i - 1], nullptr, P[i - 1], 1, Vr, P[i], ps[i], pm[i], s);
    if (e != hipSuccess) return e;
    // the max partials of this level are recomputed from the previous level
    hipLaunchKernelGGL(k_max_partials, dim3((unsigned)P[i]), dim3(256), 0, s, pm[i - 1],
                       P[i - 1], pm[i]);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const FlatFin f = fin ? *fin : FlatFin{FIN_NONE, 0.0f, nullptr, nullptr, nullptr, nullptr, nullptr};
  hipLaunchKernelGGL(k_flat_final, dim3(1), dim3(1024), 0, s, ps[L - 1], pm[L - 1], P[L - 1],
                     out2, dflags, f);
  return hipGetLastError();
}

size_t flat_reduce_pair_ws(int64_t n, int chunk_log2) { return 2 * flat_reduce_ws(n, chunk_log2); }

// Two raw fp32 leaf arrays of equal length n, reduced exactly as two
// flat_reduce calls would (same chunks, same tree), in one launch per level.
hipError_t flat_reduce_pair(const float* x0, const float* x1, int64_t n, float* out0,
                            float* out1, void* ws, int chunk_log2, int32_t* dflags,
                            hipStream_t s, const PairFin* fin, const TileMap* tm) {
  const int V = vectors_for(chunk_log2, 4);
  const int64_t C0 = int64_t(256) * 4 * V;
  const int Vr = 16;
  int64_t P[16];
  int L = levels_of(n, C0, int64_t(256) * 4 * Vr, P, 16);
  FlatPair lv[16];
  char* w = (char*)ws;
  for (int y = 0; y < 2; ++y) {
    for (int i = 0; i < L; ++i) {
      lv[i].ps[y] = (float*)w;
      lv[i].pm[y] = lv[i].ps[y] + ((P[i] + 3) & ~int64_t(3));  // 16-byte aligned
      w += align256(2 * sizeof(float) * (size_t)P[i]);
    }
  }
  lv[0].x[0] = x0;
  lv[0].x[1] = x1;
  for (int i = 1; i < L; ++i) {
    lv[i].x[0] = lv[i - 1].ps[0];
    lv[i].x[1] = lv[i - 1].ps[1];
  }
  auto leaves = [&](int i, int v, int64_t len) {
    dim3 g((unsigned)P[i], 2), b(256);
    switch (v) {
      case 1: hipLaunchKernelGGL((k_flat_leaves_pair<1>), g, b, 0, s, lv[i], len); break;
      case 2: hipLaunchKernelGGL((k_flat_leaves_pair<2>), g, b, 0, s, lv[i], len); break;
      case 4: hipLaunchKernelGGL((k_flat_leaves_pair<4>), g, b, 0, s, lv[i], len); break;
      case 8: hipLaunchKernelGGL((k_flat_leaves_pair<8>), g, b, 0, s, lv[i], len); break;
      default: hipLaunchKernelGGL((k_flat_leaves_pair<16>), g, b, 0, s, lv[i], len); break;
    }
    return hipGetLastError();
  };
  hipError_t e;
  if (tm) {
    dim3 g((unsigned)P[0], 2), b(256);
    switch (V) {
      case 1: hipLaunchKernelGGL((k_flat_leaves_pair_tiled<1>), g, b, 0, s, lv[0], n, *tm); break;
      case 2: hipLaunchKernelGGL((k_flat_leaves_pair_tiled<2>), g, b, 0, s, lv[0], n, *tm); break;
      case 4: hipLaunchKernelGGL((k_flat_leaves_pair_tiled<4>), g, b, 0, s, lv[0], n, *tm); break;
      case 8: hipLaunchKernelGGL((k_flat_leaves_pair_tiled<8>), g, b, 0, s, lv[0], n, *tm); break;
      default: hipLaunchKernelGGL((k_flat_leaves_pair_tiled<16>), g, b, 0, s, lv[0], n, *tm); break;
    }
    e = hipGetLastError();
  } else {
    e = leaves(0, V, n);
  }
  if (e != hipSuccess) return e;
  for (int i = 1; i < L; ++i) {
    if ((e = leaves(i, Vr, P[i - 1])) != hipSuccess) return e;
    hipLaunchKernelGGL(k_max_partials_pair, dim3((unsigned)P[i], 2), dim3(256), 0, s, lv[i - 1],
                       lv[i], P[i - 1]);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const PairFin f = fin ? *fin : PairFin{0, 0.0f, nullptr, nullptr, nullptr, nullptr, nullptr, 0};
  hipLaunchKernelGGL(k_flat_final_pair, dim3(2), dim3(1024), 0, s, lv[L - 1], P[L - 1], out0,
                     out1, dflags, f);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// LSQ scale from a tree sum: m = fl(S * inv_n), s = fl(m * K2), r = fl(1/s).
// --------------------------------------------------------------------------
__global__ void k_lsq_finalize(const float* sum_max, float inv_n, float* sr, float* scale,
                               float* amax) {
  float m = fmul(sum_max[0], inv_n);
  float sc = fmul(m, lsq_k2());
  float r = (sc == 0.0f) ? 0.0f : fl_div(1.0f, sc);
  sr[0] = sc;
  sr[1] = r;
  if (scale) scale[0] = sc;
  if (amax) amax[0] = sum_max[1];
}

hipError_t lsq_finalize(const float* sum_max, float inv_n, float* sr, float* scale, float* amax,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_lsq_finalize, dim3(1), dim3(1), 0, s, sum_max, inv_n, sr, scale, amax);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Elementwise codes: 16 outputs (one 16-byte store) per lane and step.
// --------------------------------------------------------------------------
template <typename T, bool COLMUL>
__global__ __launch_bounds__(256) void k_quant_flat(const T* __restrict__ x,
                                                    const float* __restrict__ cm, int64_t n,
                                                    int64_t cols, const float* __restrict__ sr,
                                                    int8_t* __restrict__ q) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int NV = 16 / E;
  const float r = sr[1];
  const int64_t groups = n / 16;
  for (int64_t gi = (int64_t)blockIdx.x * 256 + threadIdx.x; gi < groups;
       gi += (int64_t)gridDim.x * 256) {
    const int64_t i0 = gi * 16;
    uint32_t packed[4] = {0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float f[E];
      Elem<T>::unpack(ld16(x + i0 + v * E), f);
      if (COLMUL) {
        int64_t col = (i0 + v * E) % cols;
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = fmul(f[e], flush(cm[col + e]));
      }
#pragma unroll
      for (int e = 0; e < E; e += 4)
        packed[(v * E + e) >> 2] = quant_pack4(f[e], f[e + 1], f[e + 2], f[e + 3], r);
    }
    st16(q + i0, u32x4{packed[0], packed[1], packed[2], packed[3]});
  }
  // tail (n % 16 elements), handled by the first lanes of block 0
  if (blockIdx.x == 0 && threadIdx.x < (n & 15)) {
    int64_t i = groups * 16 + threadIdx.x;
    float f = Elem<T>::load1(x, i);
    if (COLMUL) f = fmul(f, flush(cm[i % cols]));
    q[i] = (int8_t)quant_code(f, r);
  }
}

hipError_t quant_flat(const void* x, int dtype, const float* col_mul, int64_t n, int64_t cols,
                      const float* sr, int8_t* q, hipStream_t s) {
  int64_t groups = n / 16;
  int64_t blocks = cdiv(groups > 0 ? groups : 1, 256);
  if (blocks > 65536) blocks = 65536;
  dim3 g((unsigned)blocks), b(256);
  if (dtype == BRQ_BF16) {
    if (col_mul) hipLaunchKernelGGL((k_quant_flat<uint16_t, true>), g, b, 0, s, (const uint16_t*)x, col_mul, n, cols, sr, q);
    else hipLaunchKernelGGL((k_quant_flat<uint16_t, false>), g, b, 0, s, (const uint16_t*)x, col_mul, n, cols, sr, q);
  } else {
    if (col_mul) hipLaunchKernelGGL((k_quant_flat<float, true>), g, b, 0, s, (const float*)x, col_mul, n, cols, sr, q);
    else hipLaunchKernelGGL((k_quant_flat<float, false>), g, b, 0, s, (const float*)x, col_mul, n, cols, sr, q);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Per-row LSQ: one wave per row, 4 rows per work-group.  Vector v of lane l
// covers columns [(64 v + l) E, + E); columns past the end are +0 leaves.
// --------------------------------------------------------------------------
// The row's V 16-byte vectors of lane `lane` (zero past cols).
template <typename T, int V>
__device__ __forceinline__ void load_row(const T* __restrict__ x, int64_t row, int64_t cols,
                                         int lane, u32x4 (&raw)[V]) {
  constexpr int E = Elem<T>::kPerVec;
  const T* xr = x + row * cols;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    raw[v] = c0 < cols ? ld16(xr + c0) : u32x4{0, 0, 0, 0};
  }
}

// Statistic, step size and codes of one row whose vectors are loaded.
template <typename T, int V>
__device__ __forceinline__ void finish_row(const u32x4 (&raw)[V], int64_t row, int64_t cols,
                                           float inv_cols, int8_t* __restrict__ q,
                                           float* __restrict__ scale, float* __restrict__ amax,
                                           int32_t* flags, int lane) {
  constexpr int E = Elem<T>::kPerVec;
  float node[V];
  float mx = 0.0f;
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float f[E];
    Elem<T>::unpack(raw[v], f);  // zero vectors past cols unpack to +0
#pragma unroll
    for (int e = 0; e < E; ++e) {
      f[e] = fabs_bits(f[e]);
      mx = fmaxf(mx, f[e]);
    }
    node[v] = wave_tree<false>(reg_tree<false, E>(f));
  }
  const float S = reg_tree<false, V>(node);
  mx = wave_max(mx);
  const float sc = fmul(fmul(S, inv_cols), lsq_k2());
  const float r = (sc == 0.0f) ? 0.0f : fl_div(1.0f, sc);
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    if (c0 >= cols) continue;
    float f[E];
    Elem<T>::unpack(raw[v], f);
    uint32_t p[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < E; e += 4) p[e >> 2] = quant_pack4(f[e], f[e + 1], f[e + 2], f[e + 3], r);
    if (E == 8) *reinterpret_cast<uint2*>(q + row * cols + c0) = make_uint2(p[0], p[1]);
    else *reinterpret_cast<uint32_t*>(q + row * cols + c0) = p[0];
  }
  if (lane == 0) {
    scale[row] = sc;
    if (amax) amax[row] = mx;
    if (!__builtin_isfinite(S)) set_flag(flags, BRQ_FLAG_NONFINITE);
  }
}

template <typename T, int V>
__device__ __forceinline__ void quant_one_row(const T* __restrict__ x, int64_t row, int64_t cols,
                                              float inv_cols, int8_t* __restrict__ q,
                                              float* __restrict__ scale,
                                              float* __restrict__ amax, int32_t* flags,
                                              int lane) {
  u32x4 raw[V];
  load_row<T, V>(x, row, cols, lane, raw);
  finish_row<T, V>(raw, row, cols, inv_cols, q, scale, amax, flags, lane);
}

template <typename T, int V>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ x, int64_t rows,
                                                    int64_t cols, float inv_cols,
                                                    int8_t* __restrict__ q,
                                                    float* __restrict__ scale,
                                                    float* __restrict__ amax, int32_t* flags) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  quant_one_row<T, V>(x, row, cols, inv_cols, q, scale, amax, flags, threadIdx.x & 63);
}

// One row over W waves of a work-group (wide rows: fewer registers per lane
// and W times the work-groups): wave wv of the row owns vectors wv V/W ..
// (wv + 1) V/W - 1, so its node is the pairwise tree over an aligned run of
// V/W of the row's V vector nodes, and the W nodes, exchanged through LDS,
// close the same tree.  Every wave of the work-group reaches the barrier
// (rows past the end take no loads and store nothing).
template <typename T, int V, int W>
__device__ __forceinline__ void quant_row_split(const T* __restrict__ x, int64_t row, bool live,
                                                int64_t cols, float inv_cols,
                                                int8_t* __restrict__ q, float* __restrict__ scale,
                                                float* __restrict__ amax, int32_t* flags,
                                                int lane, int wave, float (*red)[2]) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int VW = V / W;
  const int wv = wave % W;
  const T* xr = x + row * cols;
  u32x4 raw[VW];
  float node[VW];
  float mx = 0.0f;
#pragma unroll
  for (int v = 0; v < VW; ++v) {
    const int64_t c0 = (int64_t)((wv * VW + v) * 64 + lane) * E;
    float f[E];
    if (live && c0 < cols) {
      raw[v] = ld16(xr + c0);
      Elem<T>::unpack(raw[v], f);
    } else {
      raw[v] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < E; ++e) f[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      f[e] = fabs_bits(f[e]);
      mx = fmaxf(mx, f[e]);
    }
    node[v] = wave_tree<false>(reg_tree<false, E>(f));
  }
  const float part = reg_tree<false, VW>(node);
  mx = wave_max(mx);
  if (lane == 0) {
    red[wave][0] = part;
    red[wave][1] = mx;
  }
  __syncthreads();
  if (!live) return;
  float parts[W];
#pragma unroll
  for (int k = 0; k < W; ++k) {
    parts[k] = red[wave - wv + k][0];
    mx = fmaxf(mx, red[wave - wv + k][1]);
  }
  const float S = reg_tree<false, W>(parts);
  const float sc = fmul(fmul(S, inv_cols), lsq_k2());
  const float r = (sc == 0.0f) ? 0.0f : fl_div(1.0f, sc);
#pragma unroll
  for (int v = 0; v < VW; ++v) {
    const int64_t c0 = (int64_t)((wv * VW + v) * 64 + lane) * E;
    if (c0 >= cols) continue;
    float f[E];
    Elem<T>::unpack(raw[v], f);
    uint32_t p[2] = {0, 0};
#pragma unroll
    for (int e = 0; e < E; e += 4) p[e >> 2] = quant_pack4(f[e], f[e + 1], f[e + 2], f[e + 3], r);
    if (E == 8) *reinterpret_cast<uint2*>(q + row * cols + c0) = make_uint2(p[0], p[1]);
    else *reinterpret_cast<uint32_t*>(q + row * cols + c0) = p[0];
  }
  if (wv == 0 && lane == 0) {
    scale[row] = sc;
    if (amax) amax[row] = mx;
    if (!__builtin_isfinite(S)) set_flag(flags, BRQ_FLAG_NONFINITE);
  }
}

// tensors per grouped launch (the tables travel as kernel arguments)
constexpr int kMultiMax = 16;

// waves per row of the grouped per-row kernel
constexpr int rows_waves(int V) { return V >= 16 ? 4 : V >= 8 ? 2 : 1; }
// rows per work-group of the grouped kernel: a one-wave row takes
// kRowsPerWave rows per wave, every row's loads issued before any row's
// work, so each wave waits for memory once per kRowsPerWave rows
constexpr int kRowsPerWave = 2;
constexpr int rows_per_block(int V) {
  return rows_waves(V) == 1 ? 4 * kRowsPerWave : 4 / rows_waves(V);
}

// Several tensors' per-row quantisations in one launch: work-group b
// belongs to the tensor whose block range [start[k], start[k + 1]) holds
// it and quantises its rows rows_per_block(V) (b - start[k]) .. (two rows
// per wave when a row takes one wave, else W = rows_waves(V) waves per
// row), V the tensor's vectors per lane and row.
struct RowsJob {
  const void* x;
  int64_t rows, cols;
  int8_t* q;
  float* scale;
  float* amax;
  float inv_cols;
  int V;
};
struct RowsTable {
  RowsJob j[kMultiMax];
  int64_t start[kMultiMax + 1];
  int count;
};

template <typename T, int V>
__device__ __forceinline__ void rows_job(const RowsJob& j, int64_t blk, int wave, int lane,
                                         int32_t* flags, float (*red)[2]) {
  constexpr int W = rows_waves(V);
  if constexpr (W == 1) {
    // rows blk 4 R + wave + 4 i, i < R = kRowsPerWave
    const int64_t r0 = blk * (4 * kRowsPerWave) + wave;
    u32x4 xr[kRowsPerWave][V];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      if (r0 + 4 * i < j.rows) load_row<T, V>((const T*)j.x, r0 + 4 * i, j.cols, lane, xr[i]);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
      if (r0 + 4 * i < j.rows)
        finish_row<T, V>(xr[i], r0 + 4 * i, j.cols, j.inv_cols, j.q, j.scale, j.amax, flags,
                         lane);
  } else {
    const int64_t row = blk * (4 / W) + wave / W;
    quant_row_split<T, V, W>((const T*)j.x, row, row < j.rows, j.cols, j.inv_cols, j.q, j.scale,
                             j.amax, flags, lane, wave, red);
  }
}

// VMAX: the widest V the launch holds (its register budget); each job's V
// is dispatched at run time (uniform per work-group).
template <typename T, int VMAX>
__global__ __launch_bounds__(256) void k_quant_rows_multi(RowsTable tab, int32_t* flags) {
  __shared__ float red[4][2];
  const int64_t b = blockIdx.x;
  int k = 0;
  while (k + 1 < tab.count && b >= tab.start[k + 1]) ++k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const RowsJob& j = tab.j[k];
  const int64_t blk = b - tab.start[k];
  switch (j.V) {
    case 1: rows_job<T, 1>(j, blk, wave, lane, flags, red); break;
    case 2: rows_job<T, 2>(j, blk, wave, lane, flags, red); break;
    case 4: rows_job<T, 4>(j, blk, wave, lane, flags, red); break;
    case 8: if constexpr (VMAX >= 8) rows_job<T, 8>(j, blk, wave, lane, flags, red); break;
    case 16: if constexpr (VMAX >= 16) rows_job<T, 16>(j, blk, wave, lane, flags, red); break;
    case 32: if constexpr (VMAX >= 32) rows_job<T, 32>(j, blk, wave, lane, flags, red); break;
    default: if constexpr (VMAX >= 64) rows_job<T, 64>(j, blk, wave, lane, flags, red); break;
  }
}

// vectors of 16 bytes per lane and row: the power of two covering cols
int rows_vectors(int dtype, int64_t cols) {
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  const int64_t per = (cols + 64 * E - 1) / (64 * E);
  int V = 1;
  while (V < per) V *= 2;
  return V;
}

hipError_t quant_rows(const void* x, int dtype, int64_t rows, int64_t cols, int8_t* q,
                      float* scale, float* amax, int32_t* dflags, hipStream_t s) {
  const int V = rows_vectors(dtype, cols);
  const float inv_cols = 1.0f / (float)cols;  // host binary32 division, correctly rounded
  dim3 g((unsigned)cdiv(rows, 4)), b(256);
#define BRQ_ROWS(TT, VV)                                                                    \
  hipLaunchKernelGGL((k_quant_rows<TT, VV>), g, b, 0, s, (const TT*)x, rows, cols, inv_cols, q, \
                     scale, amax, dflags)
  if (dtype == BRQ_BF16) {
    switch (V) {
      case 1: BRQ_ROWS(uint16_t, 1); break;
      case 2: BRQ_ROWS(uint16_t, 2); break;
      case 4: BRQ_ROWS(uint16_t, 4); break;
      case 8: BRQ_ROWS(uint16_t, 8); break;
      case 16: BRQ_ROWS(uint16_t, 16); break;
      default: BRQ_ROWS(uint16_t, 32); break;
    }
  } else {
    switch (V) {
      case 1: BRQ_ROWS(float, 1); break;
      case 2: BRQ_ROWS(float, 2); break;
      case 4: BRQ_ROWS(float, 4); break;
      case 8: BRQ_ROWS(float, 8); break;
      case 16: BRQ_ROWS(float, 16); break;
      case 32: BRQ_ROWS(float, 32); break;
      default: BRQ_ROWS(float, 64); break;
    }
  }
#undef BRQ_ROWS
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// int8 transpose through LDS, 64x64 tiles.  rows % 16 == 0, cols % 16 == 0.
// --------------------------------------------------------------------------
__device__ __forceinline__ void transpose_tile(const int8_t* __restrict__ q, int64_t rows,
                                               int64_t cols, int8_t* __restrict__ qt, int64_t r0,
                                               int64_t c0) {
  __shared__ uint32_t tile[64][17];  // 64 rows x 64 bytes, one padding word per row
  const int t = threadIdx.x;
  {
    const int r = t >> 2, ch = t & 3;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < rows && c0 + ch * 16 < cols) v = ld16(q + (r0 + r) * cols + c0 + ch * 16);
    tile[r][ch * 4 + 0] = v.x;
    tile[r][ch * 4 + 1] = v.y;
    tile[r][ch * 4 + 2] = v.z;
    tile[r][ch * 4 + 3] = v.w;
  }
  __syncthreads();
  const int c = t >> 2, rg = (t & 3) * 16;  // output row c (input column), 16 input rows
  if (c0 + c >= cols || r0 + rg >= rows) return;
  uint32_t p[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t word = tile[rg + i][c >> 2];
    uint32_t byte = (word >> (8 * (c & 3))) & 0xffu;
    p[i >> 2] |= byte << (8 * (i & 3));
  }
  st16(qt + (c0 + c) * rows + r0 + rg, u32x4{p[0], p[1], p[2], p[3]});
}

__global__ __launch_bounds__(256) void k_transpose_i8(const int8_t* __restrict__ q, int64_t rows,
                                                      int64_t cols, int8_t* __restrict__ qt) {
  transpose_tile(q, rows, cols, qt, (int64_t)blockIdx.y * 64, (int64_t)blockIdx.x * 64);
}

// 128 x 128 tile per work-group (16 KiB each way): each lane loads four
// 16-byte pieces of input rows (8 lanes per 128-byte row), and each store
// writes 16 bytes of one output row, 8 neighbouring lanes covering an
// output row's 128 bytes.  rows % 16 == 0 and cols % 16 == 0 (whole
// 16-byte pieces).
__device__ __forceinline__ void transpose_tile128(const int8_t* __restrict__ q, int64_t rows,
                                                  int64_t cols, int8_t* __restrict__ qt,
                                                  int64_t r0, int64_t c0) {
  __shared__ uint32_t tile[128][33];  // 128 rows x 128 bytes, one padding word per row
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + t, r = id >> 3, ch = id & 7;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < rows && c0 + ch * 16 < cols) v = ld16(q + (r0 + r) * cols + c0 + ch * 16);
    tile[r][ch * 4 + 0] = v.x;
    tile[r][ch * 4 + 1] = v.y;
    tile[r][ch * 4 + 2] = v.z;
    tile[r][ch * 4 + 3] = v.w;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int id = i * 256 + t, c = id >> 3, rg = (id & 7) * 16;
    if (c0 + c >= cols || r0 + rg >= rows) continue;
    uint32_t p[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t byte = (tile[rg + k][c >> 2] >> (8 * (c & 3))) & 0xffu;
      p[k >> 2] |= byte << (8 * (k & 3));
    }
    st16(qt + (c0 + c) * rows + r0 + rg, u32x4{p[0], p[1], p[2], p[3]});
  }
}

// Several transposes in one launch: work-group b is tile b - start[k] of
// tensor k (tiles_x tiles of 128 x 128 per row of tiles).
struct TrJob {
  const int8_t* q;
  int64_t rows, cols;
  int8_t* qt;
  int64_t tiles_x;
};
struct TrTable {
  TrJob j[kMultiMax];
  int64_t start[kMultiMax + 1];
  int count;
};

__global__ __launch_bounds__(256) void k_transpose_i8_multi(TrTable tab) {
  const int64_t b = blockIdx.x;
  int k = 0;
  while (k + 1 < tab.count && b >= tab.start[k + 1]) ++k;
  const int64_t tile = b - tab.start[k], tx = tab.j[k].tiles_x;
  const int64_t by = tile / tx, bx = tile - by * tx;
  transpose_tile128(tab.j[k].q, tab.j[k].rows, tab.j[k].cols, tab.j[k].qt, by * 128, bx * 128);
}

hipError_t transpose_i8(const int8_t* q, int64_t rows, int64_t cols, int8_t* qt, hipStream_t s) {
  dim3 g((unsigned)cdiv(cols, 64), (unsigned)cdiv(rows, 64)), b(256);
  hipLaunchKernelGGL(k_transpose_i8, g, b, 0, s, q, rows, cols, qt);
  return hipGetLastError();
}

// Per-row quantisation of several tensors (with transposed codes where
// asked): one launch per table of up to kMultiMax tensors of one element
// type and width class (rows up to 16 vectors a lane, or one wider V),
// then one launch per table of transposes.
hipError_t quant_rows_multi(const brq_rows_job* jobs, int count, int32_t* dflags, hipStream_t s) {
  bool done[BRQ_ROWS_MULTI_MAX] = {};
  for (int a = 0; a < count; ++a) {
    if (done[a]) continue;
    const int dtype = jobs[a].x_dtype;
    // one launch class for every V up to 16 (at most 67 registers a lane),
    // one per wider V
    auto vclass = [&](int64_t cols) {
      const int V = rows_vectors(dtype, cols);
      return V <= 16 ? 16 : V;
    };
    const int VC = vclass(jobs[a].cols);
    RowsTable tab{};
    int64_t blocks = 0;
    auto flush_table = [&]() -> hipError_t {
      if (tab.count == 0) return hipSuccess;
      tab.start[tab.count] = blocks;
      dim3 g((unsigned)blocks), b(256);
#define BRQ_MULTI(TT, VV) hipLaunchKernelGGL((k_quant_rows_multi<TT, VV>), g, b, 0, s, tab, dflags)
      if (dtype == BRQ_BF16) {
        if (VC == 16) BRQ_MULTI(uint16_t, 16);
        else BRQ_MULTI(uint16_t, 32);
      } else {
        if (VC == 16) BRQ_MULTI(float, 16);
        else if (VC == 32) BRQ_MULTI(float, 32);
        else BRQ_MULTI(float, 64);
      }
#undef BRQ_MULTI
      tab = RowsTable{};
      blocks = 0;
      return hipGetLastError();
    };
    for (int c = a; c < count; ++c) {
      if (done[c] || jobs[c].x_dtype != dtype || vclass(jobs[c].cols) != VC) continue;
      done[c] = true;
      if (jobs[c].rows == 0) continue;
      RowsJob& j = tab.j[tab.count];
      j.x = jobs[c].x;
      j.rows = jobs[c].rows;
      j.cols = jobs[c].cols;
      j.q = jobs[c].q;
      j.scale = jobs[c].scale;
      j.amax = jobs[c].amax;
      j.inv_cols = 1.0f / (float)jobs[c].cols;  // host binary32 division, correctly rounded
      j.V = rows_vectors(dtype, jobs[c].cols);
      tab.start[tab.count] = blocks;
      blocks += cdiv(jobs[c].rows, rows_per_block(j.V));
      if (++tab.count == kMultiMax) {
        const hipError_t e = flush_table();
        if (e != hipSuccess) return e;
      }
    }
    const hipError_t e = flush_table();
    if (e != hipSuccess) return e;
  }
  TrTable tt{};
  int64_t tblocks = 0;
  auto flush_tr = [&]() -> hipError_t {
    if (tt.count == 0) return hipSuccess;
    tt.start[tt.count] = tblocks;
    hipLaunchKernelGGL(k_transpose_i8_multi, dim3((unsigned)tblocks), dim3(256), 0, s, tt);
    tt = TrTable{};
    tblocks = 0;
    return hipGetLastError();
  };
  for (int c = 0; c < count; ++c) {
    if (!jobs[c].q_t || jobs[c].rows == 0) continue;
    TrJob& j = tt.j[tt.count];
    j.q = jobs[c].q;
    j.rows = jobs[c].rows;
    j.cols = jobs[c].cols;
    j.qt = jobs[c].q_t;
    j.tiles_x = cdiv(jobs[c].cols, 128);
    tt.start[tt.count] = tblocks;
    tblocks += j.tiles_x * cdiv(jobs[c].rows, 128);
    if (++tt.count == kMultiMax) {
      const hipError_t e = flush_tr();
      if (e != hipSuccess) return e;
    }
  }
  return flush_tr();
}

}  // namespace brq
