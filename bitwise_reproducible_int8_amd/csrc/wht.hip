// wht.hip -- Walsh-Hadamard rotation along tokens before the int8 weight-
// gradient GEMM (Open-1B report §3.2 "int8 computation": a Walsh-Hadamard
// rotation along the contraction dimension flattens gradient outliers
// before int8 quantisation).  H_b is the unnormalised Sylvester matrix,
// H[i][j] = (-1)^popcount(i & j), applied to each aligned block of b
// tokens; the 1/b of H^T H = b I is folded into the dW epilogue.
//
// Both rotated tensors are written transposed (token-contiguous) so the dW
// GEMM reads its contraction dimension contiguously.
//
// Integer side: u = H q_x is exact (|u| <= 127 b fits int16), so two
// columns ride in one register as packed int16 lanes, and the statistic
// sum |u| is an exact integer (any order).
//
// Float side: v is computed by butterflies in stage order h = 1, 2, ...,
// b/2, each (v_j, v_j+h) <- (fl(v_j + v_j+h), fl(v_j - v_j+h)) -- the
// rounding sequence the definition fixes -- one column per lane, all b
// tokens in registers.  Its per-tensor statistic is the canonical tree over
// |v| in row-major [M][N] order: each wave owns 64 aligned columns, so for
// every token row it produces node(6, .) of the row-major tree (an LDS
// transpose gives each lane 16 consecutive columns of one row; the lane
// quad then pairs up), and the flat tree reduction finishes the job.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

typedef short s16x2 __attribute__((ext_vector_type(2)));

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- integer rotation ---------------------------------------------------------
// A work-group owns a tile of TB tokens x 512 columns of q_x.  The tile goes
// from global memory straight into LDS (global_load_lds_dwordx4, row-major
// 16-byte chunks: chunk c holds row c / 32, columns 16 (c % 32) .. + 15;
// wave w's load i fills chunks 256 i + 64 w + lane), so every global load
// reads whole 512-byte row segments.  Thread t then takes columns 2t and
// 2t + 1 of every row from LDS as one packed pair of int16 lanes and runs
// the butterflies in registers.  Chunks past K read a clamped in-bounds
// chunk whose columns are never used.
constexpr int kWhtCols = 512;

template <int TB>
__device__ __forceinline__ void wht_tile_load(const int8_t* __restrict__ q_x, int64_t K,
                                              int64_t m0, int64_t k0, int8_t* tile) {
  const int t = threadIdx.x, wave = t >> 6;
  // load i of thread t: row 8 i + t / 32, the same columns for every i
  int64_t col = k0 + (t % (kWhtCols / 16)) * 16;
  col = col < K ? col : k0;
  const int8_t* src = q_x + (m0 + t / (kWhtCols / 16)) * K + col;
  const int64_t step = (int64_t)(256 / (kWhtCols / 16)) * K;
#pragma unroll
  for (int i = 0; i < TB * (kWhtCols / 16) / 256; ++i, src += step) {
    __builtin_amdgcn_global_load_lds(
        (const void*)src,
        (__attribute__((address_space(3))) void*)(tile + (i * 256 + wave * 64) * 16), 16, 0, 0);
  }
  // every load of the tile has landed (this wave's), then every wave's
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
  __syncthreads();
}

template <int TB>
__device__ __forceinline__ void load_int_cols(const int8_t* tile, s16x2* u) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < TB; ++i) {
    const uint32_t w = *reinterpret_cast<const uint16_t*>(tile + i * kWhtCols + 2 * t);
    // bytes (0, c0, 0, c1), then an arithmetic shift of each 16-bit half by 8
    const uint32_t hi = __builtin_amdgcn_perm(w, w, 0x010c000cu);
    u[i] = __builtin_bit_cast(s16x2, hi) >> (s16x2){8, 8};
  }
}

template <int TB, typename V>
__device__ __forceinline__ void butterflies_int(V* u, int b) {
#pragma unroll
  for (int h = 1; h < TB; h *= 2) {
    if (h < b) {
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if (j & h) continue;
        // in place, two instructions and no temporary: s = a + c, then
        // a - c as c * -2 + s (v_pk_mad_i16; every value and partial sum
        // fits 16 bits, so the wrapped product sum is the exact difference)
        const V sum = u[j] + u[j + h];
        V dif;
        asm("v_pk_mad_i16 %0, %1, %2, %3" : "=v"(dif) : "v"(u[j + h]), "v"(0xfffefffeu), "v"(sum));
        u[j] = sum;
        u[j + h] = dif;
      }
    }
  }
}

// Pass 1 on a tile already in LDS: sum |u| over the work-group's tile
// (one int64 partial per work-group).
template <int TB>
__device__ __forceinline__ void wht_int_stats_tile(const int8_t* tile, int64_t K, int64_t k0,
                                                   int b, long long* __restrict__ part) {
  const int64_t k = k0 + 2 * threadIdx.x;
  int s = 0;
  if (k < K) {
    s16x2 u[TB];
    load_int_cols<TB>(tile, u);
    butterflies_int<TB>(u, b);
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      // |u| <= 127 * 128 fits both halves; the dot with (1, 1) adds them
      const s16x2 a = __builtin_elementwise_max(u[i], -u[i]);
      s = __builtin_amdgcn_sdot2(a, (s16x2){1, 1}, s, false);
    }
  }
  // integer sums: exact in any order
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  __shared__ int ws[4];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0)
    part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] =
        (long long)ws[0] + ws[1] + ws[2] + ws[3];
}

// Pass 1: sum |u| per work-group (int64 partials).
template <int TB>
__global__ __launch_bounds__(256) void k_wht_int_stats(const int8_t* __restrict__ q_x, int64_t M,
                                                       int64_t K, int b,
                                                       long long* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) int8_t tile[TB * kWhtCols];
  const int64_t k0 = (int64_t)blockIdx.x * kWhtCols;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  wht_tile_load<TB>(q_x, K, m0, k0, tile);
  wht_int_stats_tile<TB>(tile, K, k0, b, part);
}

// The activation codes and pass 1 in one kernel: the work-group quantises
// its TB x 512 tile of x (the per-tensor LSQ codes, exactly as k_quant_flat
// forms them: DAZ, fl(v * r), clamp, round half to even), writes them to
// q_x row by row, and keeps them in LDS in the layout wht_tile_load gives,
// so pass 1 needs no read of q_x.  Lane t quantises 16 elements of one row
// per step (32 lanes per 512-column row segment); columns past K are zero
// codes in LDS and are never used.  K % 16 == 0.
template <typename T, int TB>
__global__ __launch_bounds__(256) void k_quant_x_wht(const T* __restrict__ x, int64_t M,
                                                     int64_t K, int b,
                                                     const float* __restrict__ sr,
                                                     int8_t* __restrict__ q,
                                                     long long* __restrict__ part) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int NV = 16 / E;
  __shared__ __attribute__((aligned(1024))) int8_t tile[TB * kWhtCols];
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kWhtCols;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  const float r = sr[1];
  // chunk i of thread t: row 8 i + t / 32, the same columns for every i
  const int64_t col = k0 + (t % (kWhtCols / 16)) * 16;
  const int64_t rstep = (int64_t)(256 / (kWhtCols / 16)) * K;
  const T* src = x + (m0 + t / (kWhtCols / 16)) * K + col;
  int8_t* dst = q + (m0 + t / (kWhtCols / 16)) * K + col;
#pragma unroll 4
  for (int i = 0; i < TB * (kWhtCols / 16) / 256; ++i, src += rstep, dst += rstep) {
    const int c = i * 256 + t;
    uint32_t packed[4] = {0, 0, 0, 0};
    if (col < K) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        float f[E];
        Elem<T>::unpack(ld16(src + v * E), f);
#pragma unroll
        for (int e = 0; e < E; e += 4)
          packed[(v * E + e) >> 2] = quant_pack4(f[e], f[e + 1], f[e + 2], f[e + 3], r);
      }
      st16(dst, u32x4{packed[0], packed[1], packed[2], packed[3]});
    }
    st16(tile + (int64_t)c * 16, u32x4{packed[0], packed[1], packed[2], packed[3]});
  }
  __syncthreads();
  wht_int_stats_tile<TB>(tile, K, k0, b, part);
}

// Exact total, then the LSQ step: fl(double(S)) -> fl(* inv_n) -> fl(* K2).
__global__ __launch_bounds__(256) void k_wht_int_finalize(const long long* __restrict__ part,
                                                          int64_t P, float inv_n, float* sr,
                                                          float* s_out) {
  long long s = 0;
  for (int64_t i = threadIdx.x; i < P; i += 256) s += part[i];
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  __shared__ long long ws[4];
  if ((threadIdx.x & 63) == 0) ws[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    long long S = ws[0] + ws[1] + ws[2] + ws[3];
    float Sf = (float)(double)S;  // exact in double (S < 2^53), one rounding
    float sc = fmul(fmul(Sf, inv_n), lsq_k2());
    float r = (sc == 0.0f) ? 0.0f : fl_div(1.0f, sc);
    sr[0] = sc;
    sr[1] = r;
    if (s_out) s_out[0] = sc;
  }
}

// Pass 2: recompute u, quantise, write q_u^T [K][M].  The codes go through
// the same LDS tile transposed, [512 columns][TB tokens], 16-token chunks
// XOR-swizzled by column (the 8 lanes of one LDS access cycle write 8
// different bank groups), so that each global store instruction writes
// whole TB-byte column runs: 16 bytes per lane, TB / 16 lanes per column.
template <int TB>
__global__ __launch_bounds__(256) void k_wht_int_quant(const int8_t* __restrict__ q_x, int64_t M,
                                                       int64_t K, int b, const float* __restrict__ sr,
                                                       int8_t* __restrict__ q_ut) {
  constexpr int QC = TB / 16;  // 16-token chunks per column
  __shared__ __attribute__((aligned(1024))) int8_t tile[TB * kWhtCols];
  const int t = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * kWhtCols;
  const int64_t k = k0 + 2 * t;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  const float r = sr[1];
  wht_tile_load<TB>(q_x, K, m0, k0, tile);
  s16x2 u[TB];
  load_int_cols<TB>(tile, u);
  butterflies_int<TB>(u, b);
  // every thread has read its columns: the tile takes the codes
  __syncthreads();
  if (k < K) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int cc = 2 * t + c;
#pragma unroll
      for (int p = 0; p < QC; ++p) {
        uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          float f[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = (float)(c ? u[16 * p + i + e].y : u[16 * p + i + e].x);
          w[i >> 2] = quant_pack4(f[0], f[1], f[2], f[3], r);
        }
        st16(tile + cc * TB + ((p ^ ((cc >> 1) & (QC - 1))) * 16), u32x4{w[0], w[1], w[2], w[3]});
      }
    }
  }
  __syncthreads();
  // store j of thread t: column (256 / QC) j + t / QC, the same tokens for
  // every j, so the destination steps by (256 / QC) M
  int8_t* dst = q_ut + (k0 + t / QC) * M + m0 + 16 * (t % QC);
  const int64_t dstep = (int64_t)(256 / QC) * M;
#pragma unroll
  for (int j = 0; j < kWhtCols * QC / 256; ++j, dst += dstep) {
    const int ch = j * 256 + t;
    const int cc = ch / QC, q = ch % QC;
    if (k0 + cc >= K) continue;
    st16(dst, ld16(tile + cc * TB + ((q ^ ((cc >> 1) & (QC - 1))) * 16)));
  }
}

size_t wht_x_ws(int64_t M, int64_t K, int block) {
  const int TB = block > 64 ? 128 : 64;
  int64_t P = cdiv(K, kWhtCols) * (M / TB);
  return align256((size_t)(P > 0 ? P : 1) * sizeof(long long)) + 256;
}

// s = 0: the step size of an empty group (no mean is taken)
__global__ void k_step_zero(float* s_out) { s_out[0] = 0.0f; }

hipError_t wht_quant_x(const int8_t* q_x, int64_t M, int64_t K, int block, int8_t* q_ut,
                       float* s_u, void* ws, hipStream_t s) {
  if (M == 0 || K == 0) {
    hipLaunchKernelGGL(k_step_zero, dim3(1), dim3(1), 0, s, s_u);
    return hipGetLastError();
  }
  const int TB = block > 64 ? 128 : 64;
  dim3 g((unsigned)cdiv(K, kWhtCols), (unsigned)(M / TB)), bl(256);
  const int64_t P = (int64_t)g.x * g.y;
  long long* part = (long long*)ws;
  float* sr = (float*)((char*)ws + align256((size_t)(P > 0 ? P : 1) * sizeof(long long)));
  const float inv_n = 1.0f / (float)(M * K);
  if (TB == 128) hipLaunchKernelGGL(k_wht_int_stats<128>, g, bl, 0, s, q_x, M, K, block, part);
  else hipLaunchKernelGGL(k_wht_int_stats<64>, g, bl, 0, s, q_x, M, K, block, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_wht_int_finalize, dim3(1), dim3(256), 0, s, part, P, inv_n, sr, s_u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (TB == 128) hipLaunchKernelGGL(k_wht_int_quant<128>, g, bl, 0, s, q_x, M, K, block, sr, q_ut);
  else hipLaunchKernelGGL(k_wht_int_quant<64>, g, bl, 0, s, q_x, M, K, block, sr, q_ut);
  return hipGetLastError();
}

// The activation codes with the integer rotation of those codes, in one
// call: the per-tensor statistic of x (tree, step size formed by the final
// work-group), the codes and the rotation's pass 1 from one read of x
// (k_quant_x_wht), then the rotation's step size and pass 2.  The results
// are those of quantize_lsq (per tensor) followed by wht_quant_x on its
// codes; the statistic pass over q_x is the read this saves.
size_t quant_x_wht_ws(int64_t M, int64_t K, int block, int chunk_log2) {
  return align256(flat_reduce_ws(M * K, chunk_log2) + 256) + wht_x_ws(M, K, block);
}

hipError_t quantize_x_wht(const void* x, int dtype, int64_t M, int64_t K, int block,
                          int8_t* q_x, float* s_x, float* amax_x, int8_t* q_ut, float* s_u,
                          void* ws, int chunk_log2, int32_t* dflags, hipStream_t s) {
  const int64_t n = M * K;
  char* w = (char*)ws;
  const size_t fsz = flat_reduce_ws(n, chunk_log2);
  float* sc = (float*)(w + fsz);  // [0] sum [1] max [2] s [3] r
  void* wws = w + align256(fsz + 256);
  // an empty tensor has step size 0 (no mean is taken)
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;  // host binary32 division
  const FlatFin fin{FIN_LSQ, inv_n, sc + 2, s_x, amax_x, nullptr, nullptr};
  hipError_t e = flat_reduce(x, dtype, LEAF_ABS, nullptr, n, K > 0 ? K : 1, sc, w, chunk_log2,
                             dflags, s, 0, &fin);
  if (e != hipSuccess) return e;
  if (n == 0) return wht_quant_x(q_x, M, K, block, q_ut, s_u, wws, s);
  const int TB = block > 64 ? 128 : 64;
  dim3 g((unsigned)cdiv(K, kWhtCols), (unsigned)(M / TB)), bl(256);
  const int64_t P = (int64_t)g.x * g.y;
  long long* part = (long long*)wws;
  float* sr = (float*)((char*)wws + align256((size_t)P * sizeof(long long)));
#define BRQ_QXW(TT, BB)                                                                       \
  hipLaunchKernelGGL((k_quant_x_wht<TT, BB>), g, bl, 0, s, (const TT*)x, M, K, block, sc + 2, \
                     q_x, part)
  if (dtype == BRQ_BF16) {
    if (TB == 128) BRQ_QXW(uint16_t, 128);
    else BRQ_QXW(uint16_t, 64);
  } else {
    if (TB == 128) BRQ_QXW(float, 128);
    else BRQ_QXW(float, 64);
  }
#undef BRQ_QXW
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_wht_int_finalize, dim3(1), dim3(256), 0, s, part, P,
                     1.0f / (float)(M * K), sr, s_u);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (TB == 128) hipLaunchKernelGGL(k_wht_int_quant<128>, g, bl, 0, s, q_x, M, K, block, sr, q_ut);
  else hipLaunchKernelGGL(k_wht_int_quant<64>, g, bl, 0, s, q_x, M, K, block, sr, q_ut);
  return hipGetLastError();
}

// ---- fp32 rotation ------------------------------------------------------------------
template <typename T, int TB>
__device__ __forceinline__ void load_fp_col(const T* __restrict__ dy, int64_t N, int64_t m0,
                                            int64_t col, float* v) {
#pragma unroll
  for (int i = 0; i < TB; ++i) v[i] = Elem<T>::load1(dy, (m0 + i) * N + col);
}

template <int TB>
__device__ __forceinline__ void butterflies_fp(float* v, int b) {
#pragma unroll
  for (int h = 1; h < TB; h *= 2) {
    if (h < b) {
#pragma unroll
      for (int j = 0; j < TB; ++j) {
        if (j & h) continue;
        float a = v[j], c = v[j + h];
        v[j] = fadd(a, c);
        v[j + h] = fsub(a, c);
      }
    }
  }
}

// Pass 1: node(6, .) of the row-major |v| tree for each token row of the
// tile and each wave's 64 columns: part[m * (N/64) + col/64].
template <typename T, int TB>
__global__ __launch_bounds__(256) void k_wht_fp_stats(const T* __restrict__ dy, int64_t M,
                                                      int64_t N, int b, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float tr[4][16][68];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  const bool live = col < N;  // N % 64 == 0: whole waves are live or not
  float v[TB];
  if (live) {
    load_fp_col<T, TB>(dy, N, m0, col, v);
    butterflies_fp<TB>(v, b);
  } else {
#pragma unroll
    for (int i = 0; i < TB; ++i) v[i] = 0.0f;
  }
  const int64_t nb = N / 64;
  const int64_t cb = ((int64_t)blockIdx.x * 256 + wave * 64) / 64;
#pragma unroll
  for (int p = 0; p < TB / 16; ++p) {
#pragma unroll
    for (int i = 0; i < 16; ++i) tr[wave][i][lane] = fabs_bits(v[16 * p + i]);
    __syncthreads();
    const int r = lane >> 2, c16 = (lane & 3) * 16;
    float a[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 x4 = *reinterpret_cast<const float4*>(&tr[wave][r][c16 + 4 * q]);
      a[4 * q] = x4.x; a[4 * q + 1] = x4.y; a[4 * q + 2] = x4.z; a[4 * q + 3] = x4.w;
    }
    float node = reg_tree<false, 16>(a);
    node = node + dpp_xor1(node);  // non-negative: no flush needed
    node = node + dpp_xor2(node);
    if (live && (lane & 3) == 0) part[(m0 + 16 * p + r) * nb + cb] = node;
    __syncthreads();
  }
}

// Pass 2: recompute v, quantise with r_v, write q_v^T [N][M].
template <typename T, int TB>
__global__ __launch_bounds__(256) void k_wht_fp_quant(const T* __restrict__ dy, int64_t M,
                                                      int64_t N, int b, const float* __restrict__ sr,
                                                      int8_t* __restrict__ q_vt) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.y * TB;
  if (col >= N) return;
  const float r = sr[1];
  float v[TB];
  load_fp_col<T, TB>(dy, N, m0, col, v);
  butterflies_fp<TB>(v, b);
#pragma unroll
  for (int p = 0; p < TB / 16; ++p) {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      w[i >> 2] = quant_pack4(v[16 * p + i], v[16 * p + i + 1], v[16 * p + i + 2], v[16 * p + i + 3], r);
    st16(q_vt + col * M + m0 + 16 * p, u32x4{w[0], w[1], w[2], w[3]});
  }
}

size_t wht_dy_ws(int64_t M, int64_t N, int block, int chunk_log2) {
  (void)block;
  const int64_t P = M * (N / 64);
  return align256((size_t)(P > 0 ? P : 1) * sizeof(float)) + flat_reduce_ws(P, chunk_log2) + 256;
}

hipError_t wht_quant_dy(const void* dy, int dtype, int64_t M, int64_t N, int block, int8_t* q_vt,
                        float* s_v, void* ws, int chunk_log2, int32_t* dflags, hipStream_t s) {
  const int TB = block > 64 ? 128 : 64;
  const int64_t P = M * (N / 64);
  char* w = (char*)ws;
  float* part = (float*)w;
  w += align256((size_t)(P > 0 ? P : 1) * sizeof(float));
  void* fws = w;
  w += flat_reduce_ws(P, chunk_log2);
  float* sum2 = (float*)w;  // [0] sum, [1] max, [2] s, [3] r
  float* sr = sum2 + 2;
  dim3 g((unsigned)cdiv(N, 256), (unsigned)(M / TB)), bl(256);
#define BRQ_FP(KERN, ...)                                                                         \
  do {                                                                                           \
    if (dtype == BRQ_BF16) {                                                                     \
      if (TB == 128) hipLaunchKernelGGL((KERN<uint16_t, 128>), g, bl, 0, s, (const uint16_t*)dy, \
                                        M, N, block, __VA_ARGS__);                               \
      else hipLaunchKernelGGL((KERN<uint16_t, 64>), g, bl, 0, s, (const uint16_t*)dy, M, N,      \
                              block, __VA_ARGS__);                                               \
    } else {                                                                                     \
      if (TB == 128) hipLaunchKernelGGL((KERN<float, 128>), g, bl, 0, s, (const float*)dy, M, N, \
                                        block, __VA_ARGS__);                                     \
      else hipLaunchKernelGGL((KERN<float, 64>), g, bl, 0, s, (const float*)dy, M, N, block,     \
                              __VA_ARGS__);                                                      \
    }                                                                                            \
  } while (0)
  BRQ_FP(k_wht_fp_stats, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const FlatFin fin{FIN_LSQ, 1.0f / (float)(M * N), sr, s_v, nullptr, nullptr, nullptr};
  if ((e = flat_reduce(part, BRQ_F32, LEAF_RAW, nullptr, P, 1, sum2, fws, chunk_log2, dflags, s, 0,
                       &fin)) != hipSuccess)
    return e;
  BRQ_FP(k_wht_fp_quant, sr, q_vt);
#undef BRQ_FP
  return hipGetLastError();
}

}  // namespace brq
