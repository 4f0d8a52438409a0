// exact.hip -- the LSQ step-size statistic as an exact sum (a variant of
// the quantiser of Open-1B report §3.1 "int8 quantization-aware training"
// and §3.2 "int8 computation").
//
// §3.2 makes the attention-gradient accumulation bitwise reproducible by
// summing in fixed point.  Applied to the statistic S = sum |v|: every
// binary32 value is a whole number of 2^-149 units, so S is a whole number
// N of them, and integer addition is exact in any order.  N is rounded to
// binary32 once, to nearest, ties to even; a subnormal result flushes to +0
// like every other result; a NaN input makes S NaN, otherwise an infinity
// (or a sum past the binary32 range) makes it +inf.  No step depends on the
// grid, the wave size or the order in which lanes add.
//
// Layout of N: a normal fp32 |v| = m * 2^(e-1) units, m = 2^23 + fraction
// < 2^24, e the biased exponent (1..254).  With f = e - 1 (0..253), digit
// d = f >> 4 (0..15) and shift f & 15, |v| adds m << (f & 15) (< 2^39) to
// container C[d], and N = sum_d C[d] * 2^(16 d).  A bf16 value has an 8-bit
// m, so it adds m << (f & 15) (< 2^23, one 32-bit shift) to a container
// counted in 2^16 units: its digits sit one place higher (offset 1).  Zero
// and subnormal patterns go to a seventeenth, never-read container instead
// of being masked (DAZ costs no instruction).
//
// Per-tensor groups: every work-group keeps 17 containers per thread in LDS
// (one ds_add_u64 per element, each thread its own column, so no two lanes
// contend), folds them to 16 per work-group, and one work-group adds the
// partials with 96-bit containers, composes N in 16-bit limbs and rounds.
// Per-row groups: one wave per row, the same containers per lane, folded
// and rounded inside the wave, then the codes from the values held in
// registers (one read, one write).
#include "device.hpp"
#include "internal.hpp"

namespace brq {

constexpr int kDigits = 16;
constexpr int kSlots = kDigits + 1;  // + the container of zeros and subnormals
constexpr int kLimbs = 23;  // 16-bit limbs: 17 digit places * 16 bits + 96-bit containers

// --------------------------------------------------------------------------
// One fp32 value, u = |v| as bits.  Adds its units to the thread's container
// column `col` (container d at col + d * STRIDE) and tracks the largest |v|.
// u < 2^23 (zero, subnormal: DAZ) wraps f and lands in the zero container;
// NaN and inf patterns add to digit 15, and the largest pattern then marks
// S as NaN or +inf, whatever the containers hold.
// --------------------------------------------------------------------------
template <int STRIDE>
__device__ __forceinline__ void exact_put(uint64_t* col, uint32_t u, uint32_t& umax) {
  umax = umax > u ? umax : u;
  const uint32_t f = u - 0x800000u;  // (e - 1) << 23 | fraction, for normal u
  const uint32_t d = (f >> 27) < 16u ? (f >> 27) : 16u;
  const uint32_t sh = (f >> 23) & 15u;
  const uint32_t m = (u & 0x7fffffu) | 0x800000u;
  __hip_atomic_fetch_add(col + d * STRIDE, (uint64_t)m << sh, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}

// |v| bits of one 16-byte vector: 8 bf16 or 4 fp32 values, times col_mul
// first when given (that product is one flushed binary32 multiply).
template <typename T, bool COLMUL>
__device__ __forceinline__ void abs_bits(u32x4 raw, const float* cm, int64_t col,
                                         uint32_t* u) {
  constexpr int E = Elem<T>::kPerVec;
  if (COLMUL) {
    float f[E];
    Elem<T>::unpack(raw, f);
#pragma unroll
    for (int e = 0; e < E; ++e) u[e] = __float_as_uint(fmul(f[e], flush(cm[col + e]))) & 0x7fffffffu;
  } else if (E == 8) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u[2 * k] = (w[k] << 16) & 0x7fffffffu;
      u[2 * k + 1] = w[k] & 0x7fff0000u;
    }
  } else {
    u[0] = raw.x & 0x7fffffffu;
    u[1] = raw.y & 0x7fffffffu;
    u[2] = raw.z & 0x7fffffffu;
    u[3] = raw.w & 0x7fffffffu;
  }
}

// One bf16 value, h = |v| as its 16 bits: the same with an 8-bit m, in
// containers of 2^16 units.
template <int STRIDE>
__device__ __forceinline__ void exact_put16(uint64_t* col, uint32_t h, uint32_t& hmax) {
  static_assert(STRIDE == 64 || STRIDE == 256, "container stride");
  hmax = hmax > h ? hmax : h;
  const uint32_t f = h - 0x80u;  // (e - 1) << 7 | fraction, for normal h
  // byte offset of container min(f >> 11, 16): (f >> 11) * 8 * STRIDE
  const uint32_t off = (min(f, 0x8000u) & 0xf800u) >> (STRIDE == 256 ? 0 : 2);
  const uint32_t sh = (f >> 7) & 15u;
  const uint32_t m = (h & 0x7fu) | 0x80u;
  __hip_atomic_fetch_add((uint64_t*)((char*)col + off), (uint64_t)(m << sh), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_WORKGROUP);
}

// All values of one 16-byte vector.  bf16 without a multiplier takes the
// 16-bit path; with col_mul each value is first one flushed binary32
// multiply.  `hmax` collects bf16 patterns, `umax` fp32 ones.
template <typename T, bool COLMUL, int STRIDE>
__device__ __forceinline__ void put_vec(uint64_t* col, u32x4 raw, const float* cm, int64_t c,
                                        uint32_t& umax, uint32_t& hmax) {
  if (!COLMUL && Elem<T>::kPerVec == 8) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      exact_put16<STRIDE>(col, w[k] & 0x7fffu, hmax);
      exact_put16<STRIDE>(col, (w[k] >> 16) & 0x7fffu, hmax);
    }
  } else {
    uint32_t u[Elem<T>::kPerVec];
    abs_bits<T, COLMUL>(raw, cm, c, u);
#pragma unroll
    for (int e = 0; e < Elem<T>::kPerVec; ++e) exact_put<STRIDE>(col, u[e], umax);
  }
}

// --------------------------------------------------------------------------
// N = sum_d (hi[d] * 2^64 + lo[d]) * 2^(16 (d + OFF)), rounded to binary32.
// Runs on one lane.  Column j of 16-bit limbs gathers the 16-bit pieces of
// every container that land there; the carry runs upward in 64 bits.
// --------------------------------------------------------------------------
template <int OFF>
__device__ __forceinline__ float exact_round(const uint64_t* lo, const uint32_t* hi, uint32_t umax) {
  if (umax > 0x7f800000u) return __uint_as_float(0x7fc00000u);
  if (umax == 0x7f800000u) return __uint_as_float(0x7f800000u);
  uint32_t L[kLimbs];
  uint64_t carry = 0;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
#pragma unroll
    for (int d = 0; d < kDigits; ++d) {
      const int i = j - d - OFF;  // piece i of container d: bits [16 i, 16 i + 16)
      if (i >= 0 && i < 4) carry += (lo[d] >> (16 * i)) & 0xffffu;
      else if (i >= 4 && i < 6) carry += (hi[d] >> (16 * (i - 4))) & 0xffffu;
    }
    L[j] = (uint32_t)(carry & 0xffffu);
    carry >>= 16;
  }
  // the top limb, and a 48-bit window of limbs top, top-1, top-2 (0 below 0)
  int top = -1;
  uint32_t Ltop = 0;
  uint64_t W = 0;
#pragma unroll
  for (int j = 0; j < kLimbs; ++j) {
    if (L[j] != 0u) {
      top = j;
      Ltop = L[j];
      W = ((uint64_t)L[j] << 32) | (j >= 1 ? (uint64_t)L[j - 1] << 16 : 0ull) |
          (j >= 2 ? (uint64_t)L[j - 2] : 0ull);
    }
  }
  if (top < 0) return 0.0f;
  uint32_t below = 0;  // OR of every limb under the window
#pragma unroll
  for (int j = 0; j < kLimbs; ++j)
    if (j < top - 2) below |= L[j];
  const int b = 31 - __builtin_clz(Ltop);  // top bit inside its limb
  const int topbit = 16 * top + b;
  if (topbit < 23) return 0.0f;  // N < 2^23: below 2^-126, flushed
  const int s = 9 + b;           // window position of the lowest kept bit
  uint32_t q = (uint32_t)(W >> s);
  const uint32_t half = (uint32_t)(W >> (s - 1)) & 1u;
  const bool sticky = below != 0u || (W & ((1ull << (s - 1)) - 1ull)) != 0ull;
  int lob = topbit - 23;  // N's bit index of q's lowest bit
  if (half && (sticky || (q & 1u))) {
    if (++q == (1u << 24)) {
      q >>= 1;
      ++lob;
    }
  }
  const int ef = lob + 1;  // q * 2^(lob - 149) = 1.xxx * 2^(lob - 126)
  if (ef >= 255) return __uint_as_float(0x7f800000u);
  return __uint_as_float(((uint32_t)ef << 23) | (q & 0x7fffffu));
}

// --------------------------------------------------------------------------
// Per-tensor, pass 1: work-group partials.  Grid-stride over 16-byte
// vectors, U per lane and step, the next step's loads issued before this
// step's values are added.  part[g][d] < 2^59 (a work-group sees at most
// 2^20 values: the host keeps the grid large enough).  pmax[g] is the
// largest |v| as fp32 bits.
// --------------------------------------------------------------------------
// U vectors at i0 + k * stride.  Every load is issued (an index past the end
// reads vector nvec - 1, which exists) and the caller zeroes such a vector
// when it adds it, so no branch or select sits between the loads and their
// use: the next step's loads stay in flight while this step is added.
// nvec >= 1.
template <typename T, int U>
__device__ __forceinline__ void load_step(const T* x, int64_t i0, int64_t stride, int64_t nvec,
                                          u32x4* raw) {
  constexpr int E = Elem<T>::kPerVec;
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const int64_t i = i0 + k * stride;
    raw[k] = ld16(x + (i < nvec ? i : nvec - 1) * E);
  }
}

template <typename T, bool COLMUL, int U>
__global__ __launch_bounds__(256) void k_exact_partials(const T* __restrict__ x,
                                                        const float* __restrict__ cm,
                                                        int64_t nvec, int64_t cols,
                                                        uint64_t* __restrict__ part,
                                                        uint32_t* __restrict__ pmax) {
  constexpr int E = Elem<T>::kPerVec;
  __shared__ uint64_t acc[kSlots][256];
  __shared__ uint64_t sfold[4][kDigits];
  __shared__ uint32_t smax[4];
  const int t = threadIdx.x;
#pragma unroll
  for (int d = 0; d < kSlots; ++d) acc[d][t] = 0;  // each thread's own column
  uint64_t* col = &acc[0][t];
  uint32_t umax = 0, hmax = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i0 = (int64_t)blockIdx.x * 256 + t;
  const int64_t span = stride * U;
  // col_mul columns of the U vectors, advanced by (span * E) mod cols per
  // step (one division per lane, at the start)
  int64_t c[U];
  const int64_t dspan = COLMUL ? (span * E) % cols : 0;
#pragma unroll
  for (int k = 0; k < U; ++k) c[k] = COLMUL ? ((i0 + k * stride) * E) % cols : 0;
  // a vector past the end adds zeros (its col_mul index stays in range)
  auto add_step = [&](const u32x4* raw, int64_t base) {
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const bool in = base + k * stride < nvec;
      const u32x4 v = {in ? raw[k].x : 0u, in ? raw[k].y : 0u, in ? raw[k].z : 0u,
                       in ? raw[k].w : 0u};
      put_vec<T, COLMUL, 256>(col, v, cm, c[k], umax, hmax);
      if (COLMUL) {
        c[k] += dspan;
        if (c[k] >= cols) c[k] -= cols;
      }
    }
  };
  // Two register buffers in turn: step s + 1 loads while step s adds.  The
  // step count is the same for every lane of the grid (a lane's surplus
  // vectors add zeros), so the body has no branch for the compiler to sink
  // the loads past; the scheduling barriers keep them above the adds.
  // An empty input issues no load at all (the clamped index needs nvec >= 1).
  if (nvec > 0) {
    const int64_t steps = (nvec + span - 1) / span;
    u32x4 a[U], b[U];
    load_step<T, U>(x, i0, stride, nvec, a);
    int64_t st = 0;
    for (; st + 1 < steps; st += 2) {
      load_step<T, U>(x, i0 + span, stride, nvec, b);
      __builtin_amdgcn_sched_barrier(0);
      add_step(a, i0);
      i0 += span;
      load_step<T, U>(x, i0 + span, stride, nvec, a);
      __builtin_amdgcn_sched_barrier(0);
      add_step(b, i0);
      i0 += span;
    }
    if (st < steps) add_step(a, i0);
  }
  umax = umax > (hmax << 16) ? umax : (hmax << 16);
  __syncthreads();
  // fold: thread t sums digit d = t & 15 over the 16 columns of its group
  // g = t >> 4, rotated by d so that the 64 lanes of a wave hit every bank
  // pair twice; then the 4 groups of a wave and the 4 waves combine.
  const int d = t & 15, g = t >> 4;
  uint64_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += acc[d][g * 16 + ((i + d) & 15)];
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t other = __shfl_xor(umax, o);
    umax = umax > other ? umax : other;
  }
  if ((t & 63) < 16) sfold[t >> 6][d] = sum;
  if ((t & 63) == 0) smax[t >> 6] = umax;
  __syncthreads();
  if (t < kDigits)
    part[(int64_t)blockIdx.x * kDigits + t] = (sfold[0][t] + sfold[1][t]) + (sfold[2][t] + sfold[3][t]);
  if (t == 0) {
    uint32_t m = smax[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) m = m > smax[w] ? m : smax[w];
    pmax[blockIdx.x] = m;
  }
}

// Per-tensor, pass 2: one work-group of 1024 lanes adds the G partials per
// digit with 96-bit containers (lane: digit t & 15, partials t >> 4 + 64 i,
// eight loads in flight), then one lane rounds.  out[0] = S, out[1] = max |v| (0
// when every value is zero or subnormal).  off = 1 for the bf16 containers.
__global__ __launch_bounds__(1024) void k_exact_final(const uint64_t* __restrict__ part,
                                                      const uint32_t* __restrict__ pmax,
                                                      int64_t G, int off, float* out,
                                                      int32_t* flags) {
  __shared__ uint64_t slo[64][kDigits];
  __shared__ uint32_t shi[64][kDigits], smax[16];
  const int t = threadIdx.x, d = t & 15, r = t >> 4;
  uint64_t lo = 0;
  uint32_t hi = 0;
  for (int64_t j0 = 0; j0 < G; j0 += 512) {
    uint64_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t j = j0 + r + 64 * i;
      v[i] = j < G ? part[j * kDigits + d] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo += v[i];
      hi += lo < v[i] ? 1u : 0u;
    }
  }
  uint32_t umax = 0;
  for (int64_t j = t; j < G; j += 1024) umax = umax > pmax[j] ? umax : pmax[j];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t other = __shfl_xor(umax, o);
    umax = umax > other ? umax : other;
  }
  slo[r][d] = lo;
  shi[r][d] = hi;
  if ((t & 63) == 0) smax[t >> 6] = umax;
  __syncthreads();
  if (t < kDigits) {
    uint64_t a = 0;
    uint32_t h = 0;
#pragma unroll 8
    for (int k = 0; k < 64; ++k) {
      const uint64_t w = slo[k][t];
      a += w;
      h += shi[k][t] + (a < w ? 1u : 0u);
    }
    slo[0][t] = a;
    shi[0][t] = h;
  }
  if (t == 0) {
    uint32_t m = smax[0];
    for (int k = 1; k < 16; ++k) m = m > smax[k] ? m : smax[k];
    smax[0] = m;
  }
  __syncthreads();
  if (t == 0) {
    uint64_t L[kDigits];
    uint32_t H[kDigits];
#pragma unroll
    for (int k = 0; k < kDigits; ++k) {
      L[k] = slo[0][k];
      H[k] = shi[0][k];
    }
    const uint32_t m = smax[0];
    const float S = off ? exact_round<1>(L, H, m) : exact_round<0>(L, H, m);
    out[0] = S;
    out[1] = m >= 0x800000u ? __uint_as_float(m) : 0.0f;
    if (!__builtin_isfinite(S)) set_flag(flags, BRQ_FLAG_NONFINITE);
  }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kExactU = 4;          // vectors in flight per lane
constexpr int64_t kExactMaxG = 512;  // partials (work-groups), unless n > 2^29

static int64_t exact_grid(int64_t n, int E) {
  const int64_t nvec = n / E;
  int64_t g = cdiv(nvec > 0 ? nvec : 1, 256 * kExactU);
  // at most 2^20 values per work-group keeps each partial below 2^59
  const int64_t gmin = cdiv(n > 0 ? n : 1, int64_t(1) << 20);
  if (g > kExactMaxG) g = kExactMaxG;
  if (g < gmin) g = gmin;
  return g;
}

size_t exact_reduce_ws(int64_t n) {
  const int64_t g = exact_grid(n, 4);  // fp32 gives the larger grid
  return align256((size_t)g * kDigits * sizeof(uint64_t)) + align256((size_t)g * sizeof(uint32_t));
}

hipError_t exact_reduce(const void* x, int dtype, const float* col_mul, int64_t n, int64_t cols,
                        float* out2, void* ws, int32_t* dflags, hipStream_t s) {
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  const int64_t G = exact_grid(n, E);
  uint64_t* part = (uint64_t*)ws;
  uint32_t* pmax = (uint32_t*)((char*)ws + align256((size_t)G * kDigits * sizeof(uint64_t)));
  const int64_t nvec = n / E;  // the caller guarantees cols % E == 0
  dim3 g((unsigned)G), b(256);
  if (dtype == BRQ_BF16) {
    if (col_mul)
      hipLaunchKernelGGL((k_exact_partials<uint16_t, true, kExactU>), g, b, 0, s,
                         (const uint16_t*)x, col_mul, nvec, cols, part, pmax);
    else
      hipLaunchKernelGGL((k_exact_partials<uint16_t, false, kExactU>), g, b, 0, s,
                         (const uint16_t*)x, col_mul, nvec, cols, part, pmax);
  } else {
    if (col_mul)
      hipLaunchKernelGGL((k_exact_partials<float, true, kExactU>), g, b, 0, s, (const float*)x,
                         col_mul, nvec, cols, part, pmax);
    else
      hipLaunchKernelGGL((k_exact_partials<float, false, kExactU>), g, b, 0, s, (const float*)x,
                         col_mul, nvec, cols, part, pmax);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int off = (dtype == BRQ_BF16 && !col_mul) ? 1 : 0;
  hipLaunchKernelGGL(k_exact_final, dim3(1), dim3(1024), 0, s, part, pmax, G, off, out2, dflags);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Per-row: one wave per row, 4 rows per work-group.  Vector v of lane l
// covers columns [(64 v + l) E, + E).  Containers per lane in LDS; the fold
// gives lane 4 d the row's container d (< 2^53: a row holds at most 16384
// values); lane 0 rounds.
// --------------------------------------------------------------------------
template <typename T, int V>
__global__ __launch_bounds__(256) void k_quant_rows_exact(const T* __restrict__ x, int64_t rows,
                                                          int64_t cols, float inv_cols,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale,
                                                          float* __restrict__ amax,
                                                          int32_t* flags) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int OFF = E == 8 ? 1 : 0;  // bf16 containers count 2^16 units
  __shared__ uint64_t acc[4][kSlots][64];
  __shared__ uint64_t crow[4][kDigits];
  __shared__ float srow[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const bool live = row < rows;
  const T* xr = x + (live ? row : 0) * cols;
#pragma unroll
  for (int d = 0; d < kSlots; ++d) acc[wave][d][lane] = 0;
  uint64_t* col = &acc[wave][0][lane];
  uint32_t umax = 0, hmax = 0;
  u32x4 raw[V];
#pragma unroll
  for (int v = 0; v < V; ++v) {
    const int64_t c0 = (int64_t)(v * 64 + lane) * E;
    raw[v] = (live && c0 < cols) ? ld16(xr + c0) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int v = 0; v < V; ++v) put_vec<T, false, 64>(col, raw[v], nullptr, 0, umax, hmax);
  umax = umax > (hmax << 16) ? umax : (hmax << 16);
  __syncthreads();
  {
    // lane: digit d = lane & 15 over the 16 columns of group lane >> 4,
    // rotated by d (every bank pair read twice per step)
    const int d = lane & 15, g = lane >> 4;
    uint64_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[wave][d][g * 16 + ((i + d) & 15)];
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    if (g == 0) crow[wave][d] = sum;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t other = __shfl_xor(umax, o);
    umax = umax > other ? umax : other;
  }
  __syncthreads();
  if (lane == 0) {
    uint64_t L[kDigits];
    uint32_t H[kDigits];
#pragma unroll
    for (int k = 0; k < kDigits; ++k) {
      L[k] = crow[wave][k];
      H[k] = 0;
    }
    srow[wave] = exact_round<OFF>(L, H, umax);
  }
  __syncthreads();
  if (!live) return;
  const float S = srow[wave];
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
    if (amax) amax[row] = umax >= 0x800000u ? __uint_as_float(umax) : 0.0f;
    if (!__builtin_isfinite(S)) set_flag(flags, BRQ_FLAG_NONFINITE);
  }
}

hipError_t quant_rows_exact(const void* x, int dtype, int64_t rows, int64_t cols, int8_t* q,
                            float* scale, float* amax, int32_t* dflags, hipStream_t s) {
  const int E = dtype == BRQ_BF16 ? 8 : 4;
  int64_t per = cdiv(cols, 64 * E);
  int V = 1;
  while (V < per) V *= 2;
  const float inv_cols = 1.0f / (float)cols;  // host binary32 division, correctly rounded
  dim3 g((unsigned)cdiv(rows, 4)), b(256);
#define BRQ_XROWS(TT, VV)                                                                     \
  hipLaunchKernelGGL((k_quant_rows_exact<TT, VV>), g, b, 0, s, (const TT*)x, rows, cols,       \
                     inv_cols, q, scale, amax, dflags)
  if (dtype == BRQ_BF16) {
    switch (V) {
      case 1: BRQ_XROWS(uint16_t, 1); break;
      case 2: BRQ_XROWS(uint16_t, 2); break;
      case 4: BRQ_XROWS(uint16_t, 4); break;
      case 8: BRQ_XROWS(uint16_t, 8); break;
      case 16: BRQ_XROWS(uint16_t, 16); break;
      default: BRQ_XROWS(uint16_t, 32); break;
    }
  } else {
    switch (V) {
      case 1: BRQ_XROWS(float, 1); break;
      case 2: BRQ_XROWS(float, 2); break;
      case 4: BRQ_XROWS(float, 4); break;
      case 8: BRQ_XROWS(float, 8); break;
      case 16: BRQ_XROWS(float, 16); break;
      case 32: BRQ_XROWS(float, 32); break;
      default: BRQ_XROWS(float, 64); break;
    }
  }
#undef BRQ_XROWS
  return hipGetLastError();
}

}  // namespace brq
