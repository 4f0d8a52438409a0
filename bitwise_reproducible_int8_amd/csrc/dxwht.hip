// dxwht.hip -- the input-gradient GEMM with the Walsh-Hadamard rotation
// along its contraction (a variant; Open-1B report §3.2 "int8
// computation" rotates along the contraction dimension in front of both
// straight-through gradient GEMMs).  For dX = dY * W^ the contraction runs
// over the output channels n:
//   g  = fl(dY[m][n] * s_w[n]), rotated in fp32 along each row in aligned
//        blocks of b (stage order h = 1, 2, ..., b/2), per-tensor LSQ
//        (canonical tree statistic) -> q_g, s_g
//   q_w [N][K] rotated exactly along n and requantised (the activation
//        codes' rotation, wht.hip) -> q_h^T [K][N], s_h
//   dX = fl(fl(sum_n q_g[m][n] q_h[n][k]) * fl(fl(fl(s_g * s_h) * 1) * 1/b))
// (the weight-gradient epilogue with its third scale 1: fl(x * 1) = x).
//
// The rows rotation's statistic runs in the flat tree's leaves (quant.hip,
// k_flat_leaves_wht); the codes pass below rotates again and quantises:
// each wave owns 1024 consecutive values per step, 16 per lane, so a block
// of b sits in b/16 consecutive lanes (or inside one lane).
#include "device.hpp"
#include "internal.hpp"

namespace brq {

template <typename T, int B>
__global__ __launch_bounds__(256) void k_quant_wht_rows(const T* __restrict__ x,
                                                        const float* __restrict__ cm,
                                                        int64_t nchunks, int64_t cols,
                                                        const float* __restrict__ sr,
                                                        int8_t* __restrict__ q) {
  constexpr int E = Elem<T>::kPerVec;
  constexpr int NV = 16 / E;
  const float r = sr[1];
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  // the loop bound is the same for the 64 lanes of a wave: every lane
  // reaches the cross-lane butterflies and the wave-wide fallback test
  for (int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); c < nchunks; c += nwaves) {
    const int64_t i0 = c * 1024 + lane * 16;
    const int64_t col = col_of(i0, cols);  // cols % 16 == 0: the 16 values sit in one row
    u32x4 raw[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) raw[v] = ld16(x + i0 + v * E);
    float f[16], m[16];
    uint64_t bad = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) widen_raw<T>(raw[v], f + v * E, bad);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      m[e] = cm[col + e];
      bad |= sub_mask(m[e]);
      f[e] = f[e] * m[e];
      bad |= sub_mask(f[e]);
    }
    wht_block_fast<16, B>(f, lane, bad);
    if (bad) {  // some value of the wave was subnormal: the flushed form
#pragma unroll
      for (int v = 0; v < NV; ++v) Elem<T>::unpack(raw[v], f + v * E);
#pragma unroll
      for (int e = 0; e < 16; ++e) f[e] = fmul(f[e], flush(m[e]));
      wht_block<16, B>(f, lane);
    }
    // (a subnormal product f * r rounds to code 0 with or without its flush)
    uint32_t p[4] = {0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 16; e += 4) p[e >> 2] = quant_pack4(f[e], f[e + 1], f[e + 2], f[e + 3], r);
    st16(q + i0, u32x4{p[0], p[1], p[2], p[3]});
  }
}

template <typename T>
static hipError_t launch_codes(const T* x, const float* cm, int64_t nchunks, int64_t cols, int B,
                               const float* sr, int8_t* q, hipStream_t s) {
  int64_t blocks = (nchunks + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  dim3 g((unsigned)blocks), b(256);
#define BRQ_QW(BB) hipLaunchKernelGGL((k_quant_wht_rows<T, BB>), g, b, 0, s, x, cm, nchunks, cols, sr, q)
  switch (B) {
    case 1: BRQ_QW(1); break;
    case 2: BRQ_QW(2); break;
    case 4: BRQ_QW(4); break;
    case 8: BRQ_QW(8); break;
    case 16: BRQ_QW(16); break;
    case 32: BRQ_QW(32); break;
    case 64: BRQ_QW(64); break;
    default: BRQ_QW(128); break;
  }
#undef BRQ_QW
  return hipGetLastError();
}

// sr[2] = 1: the third scale of the weight-gradient epilogue, which this
// GEMM reuses (one thread, one store)
__global__ void k_scale_one(float* sr) { sr[2] = 1.0f; }

size_t wht_rows_ws(int64_t M, int64_t N) { return flat_reduce_ws(M * N, 13) + 256; }

// q_g [M][N], s_g [1] and sr = {s_g, r_g, 1} (device) from dy [M][N] and
// s_w [N].  M * N % 1024 == 0, N % 16 == 0, N % block == 0 (checked by the
// caller).
hipError_t wht_rows_quant(const void* dy, int dtype, int64_t M, int64_t N, const float* s_w,
                          int block, int8_t* q_g, float* s_g, float* sr, void* ws,
                          int32_t* dflags, hipStream_t s) {
  const int64_t n = M * N;
  float* sc = (float*)((char*)ws + flat_reduce_ws(n, 13));  // [0] sum [1] max
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
  const FlatFin fin{FIN_LSQ, inv_n, sr, s_g, nullptr, nullptr, nullptr};
  hipError_t e =
      flat_reduce(dy, dtype, LEAF_ABS_COLMUL, s_w, n, N, sc, ws, 13, dflags, s, block, &fin);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scale_one, dim3(1), dim3(1), 0, s, sr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (n == 0) return hipSuccess;
  if (dtype == BRQ_BF16)
    return launch_codes<uint16_t>((const uint16_t*)dy, s_w, n / 1024, N, block, sr, q_g, s);
  return launch_codes<float>((const float*)dy, s_w, n / 1024, N, block, sr, q_g, s);
}

}  // namespace brq
