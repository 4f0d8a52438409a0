// gemm.hip -- W8A8 GEMMs on gfx950 matrix cores (Open-1B report §3.2 "int8
// computation": int8 x int8 products accumulated in int32, then dequantised).
//
// Every GEMM of the layer is C[i][j] = epi(sum_k A[i][k] * B[j][k]) with both
// operands contiguous along the contraction (forward: q_x, q_w; dX: q_g,
// q_w^T; dW: the token-contiguous rotated codes q_v^T, q_u^T).  The int32
// sum is exact -- 127*127*K < 2^31 for K <= 133144 -- so tile shape, MFMA
// shape, split-K and launch order cannot change a bit of it; only the
// dequantisation epilogue is floating point:
//     out = fl(fl(acc) * c_j)   one int->fp32 conversion (round to nearest
//                               even) and one multiply, flushed, no FMA.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

typedef int v4i __attribute__((ext_vector_type(4)));

struct Epi {
  int kind;
  const float* s0;
  const float* s1;
  const float* s2;
  int per_row;
  float inv_b;
  // Column scale c_j, computed in the order the definitions give.
  __device__ __forceinline__ float scale(int64_t j) const {
    if (kind == EPI_FWD) return fmul(flush(s0[0]), flush(per_row ? s1[j] : s1[0]));
    if (kind == EPI_SCALAR) return flush(s0[0]);
    return fmul(fmul(fmul(flush(s0[0]), flush(s1[0])), flush(s2[0])), inv_b);
  }
};

__device__ __forceinline__ float dequant(int acc, float c) { return fmul((float)acc, c); }

// --------------------------------------------------------------------------
// Reference kernel: one output per thread, 16-byte loads, v_dot4 products.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gemm_ref(const int8_t* __restrict__ A,
                                                  const int8_t* __restrict__ B, int64_t I,
                                                  int64_t J, int64_t Kc, float* __restrict__ C,
                                                  Epi epi) {
  const int64_t j = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  const int64_t i = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (i >= I || j >= J) return;
  const int8_t* a = A + i * Kc;
  const int8_t* b = B + j * Kc;
  int acc = 0;
  for (int64_t k = 0; k < Kc; k += 16) {
    u32x4 x = ld16(a + k), y = ld16(b + k);
    acc = __builtin_amdgcn_sdot4((int)x.x, (int)y.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)x.y, (int)y.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)x.z, (int)y.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)x.w, (int)y.w, acc, false);
  }
  C[i * J + j] = dequant(acc, epi.scale(j));
}

// --------------------------------------------------------------------------
// MFMA kernel.  Block tile BM x BN, contraction step BK = 128 bytes (one
// 128-byte line per operand row), WGM x WGN waves, each wave a
// (BM/WGM) x (BN/WGN) tile of 16x16 v_mfma_i32_16x16x64_i8 blocks.
//
// LDS holds each operand tile row-major [rows][128 B] with the 16-byte chunk
// index XOR-ed by (row >> 1) & 7, so the 16 rows one MFMA operand read
// touches spread over all banks.  Two LDS stages: while the waves multiply
// out of one stage, the next tile's global loads are in flight in registers
// and land in the other stage; one barrier per step.
//
// MFMA operand layout (16x16x64, int8): lane l supplies 16 consecutive
// contraction bytes, k-group l>>4, of row (A) or column (B) l&15; both
// operands use the same (lane, byte) -> k map, so the product sums all 64
// contraction terms.  Result: lane l holds rows 4*(l>>4)+r, column l&15.
// --------------------------------------------------------------------------
constexpr int BK = 128;

__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * BK + ((kc ^ ((row >> 1) & 7)) << 4);
}

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM* WGN * 64) void k_gemm_mfma(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t I, int64_t J,
    int64_t Kc, float* __restrict__ C, int* __restrict__ Cpart, int ktiles_per_split, Epi epi) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int LA = BM * BK / 16 / NT, LB = BN * BK / 16 / NT;
  static_assert(LA * NT * 16 == BM * BK && LB * NT * 16 == BN * BK, "tile/threads");
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // XCD-aware tile order: work-groups are dealt round-robin over the 8
  // XCDs; give each XCD a contiguous run of tiles (shared operand rows in
  // its own L2), then walk tiles in groups of 8 block-rows.
  const int64_t gm = (I + BM - 1) / BM, gn = (J + BN - 1) / BN;
  const int64_t total = gm * gn;
  int64_t pid = blockIdx.x;
  if ((total & 7) == 0) pid = (pid & 7) * (total >> 3) + (pid >> 3);
  const int64_t group = 8 * gn;
  const int64_t first_m = (pid / group) * 8;
  const int64_t gsz = (gm - first_m) < 8 ? (gm - first_m) : 8;
  const int64_t bm = first_m + (pid % group) % gsz;
  const int64_t bn = (pid % group) / gsz;
  const int64_t row0 = bm * BM, col0 = bn * BN;

  const int64_t nk_total = (Kc + BK - 1) / BK;
  const int64_t kt0 = (int64_t)blockIdx.z * ktiles_per_split;
  int64_t kt1 = kt0 + ktiles_per_split;
  if (kt1 > nk_total) kt1 = nk_total;

  u32x4 ra[LA], rb[LB];
  auto gload = [&](int64_t kt) {
    const int64_t k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = t + NT * i, r = c >> 3, kc = c & 7;
      const int64_t gr = row0 + r, gk = k0 + kc * 16;
      ra[i] = (gr < I && gk < Kc) ? ld16(A + gr * Kc + gk) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int c = t + NT * i, r = c >> 3, kc = c & 7;
      const int64_t gr = col0 + r, gk = k0 + kc * 16;
      rb[i] = (gr < J && gk < Kc) ? ld16(B + gr * Kc + gk) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = t + NT * i;
      st16(&As[st][lds_off(c >> 3, c & 7)], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int c = t + NT * i;
      st16(&Bs[st][lds_off(c >> 3, c & 7)], rb[i]);
    }
  };

  v4i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  if (kt0 < kt1) {
    gload(kt0);
    lstore(0);
    __syncthreads();
    for (int64_t kt = kt0; kt < kt1; ++kt) {
      const int st = (int)((kt - kt0) & 1);
      if (kt + 1 < kt1) gload(kt + 1);
#pragma unroll
      for (int kk = 0; kk < BK / 64; ++kk) {
        const int kc = kk * 4 + (lane >> 4);
        v4i af[TI], bf[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int r = wm * WM + i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const v4i*>(&As[st][lds_off(r, kc)]);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int r = wn * WN + j * 16 + (lane & 15);
          bf[j] = *reinterpret_cast<const v4i*>(&Bs[st][lds_off(r, kc)]);
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      if (kt + 1 < kt1) lstore(st ^ 1);
      __syncthreads();
    }
  }

  // Epilogue.  Split-K writes exact int32 partials instead.
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t col = col0 + wn * WN + j * 16 + (lane & 15);
    if (col >= J) continue;
    const float c = Cpart ? 0.0f : epi.scale(col);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + wm * WM + i * 16 + 4 * (lane >> 4) + r;
        if (row >= I) continue;
        if (Cpart) Cpart[((int64_t)blockIdx.z * I + row) * J + col] = acc[i][j][r];
        else C[row * J + col] = dequant(acc[i][j][r], c);
      }
    }
  }
}

// Sum of the split-K partials in split order (exact in int32), then the
// same epilogue.
__global__ __launch_bounds__(256) void k_splitk_reduce(const int* __restrict__ Cpart, int splits,
                                                       int64_t I, int64_t J, float* __restrict__ C,
                                                       Epi epi) {
  const int64_t n = I * J;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    int acc = 0;
    for (int z = 0; z < splits; ++z) acc += Cpart[z * n + e];
    C[e] = dequant(acc, epi.scale(e % J));
  }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int pick_kernel(const brq_tune* t) { return (t && t->gemm_kernel) ? t->gemm_kernel : 2; }
static int pick_splits(const brq_tune* t) {
  int s = (t && t->split_k) ? t->split_k : 1;
  return (s == 2 || s == 4) ? s : 1;
}

size_t gemm_ws(int64_t I, int64_t J, int64_t Kc, const brq_tune* t) {
  (void)Kc;
  int s = pick_splits(t);
  if (s == 1 || pick_kernel(t) == 1) return 0;
  return align256((size_t)s * (size_t)I * (size_t)J * sizeof(int));
}

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_mfma(const int8_t* A, const int8_t* B, int64_t I, int64_t J, int64_t Kc,
                              float* C, int* Cpart, int splits, Epi epi, hipStream_t s) {
  const int64_t tiles = cdiv(I, BM) * cdiv(J, BN);
  const int64_t nk = cdiv(Kc, BK);
  const int kps = (int)cdiv(nk, splits);
  dim3 g((unsigned)tiles, 1, (unsigned)splits), b(WGM * WGN * 64);
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN>), g, b, 0, s, A, B, I, J, Kc, C, Cpart, kps,
                     epi);
  return hipGetLastError();
}

hipError_t gemm_i8(const int8_t* A, const int8_t* B, int64_t I, int64_t J, int64_t Kc, float* C,
                   const EpiArgs& ea, void* ws, size_t ws_bytes, const brq_tune* t,
                   hipStream_t s) {
  Epi epi{ea.kind, ea.s0, ea.s1, ea.s2, ea.per_row, ea.inv_b};
  if (I == 0 || J == 0) return hipSuccess;
  const int kern = pick_kernel(t);
  if (kern == 1) {
    dim3 g((unsigned)cdiv(J, 64), (unsigned)cdiv(I, 4)), b(256);
    hipLaunchKernelGGL(k_gemm_ref, g, b, 0, s, A, B, I, J, Kc, C, epi);
    return hipGetLastError();
  }
  const int splits = pick_splits(t);
  int* part = nullptr;
  if (splits > 1) {
    if (ws_bytes < gemm_ws(I, J, Kc, t)) return hipErrorInvalidValue;
    part = (int*)ws;
  }
  hipError_t e;
  switch (kern) {
    case 3: e = launch_mfma<256, 128, 2, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 4: e = launch_mfma<128, 256, 2, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    default: e = launch_mfma<128, 128, 2, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
  }
  if (e != hipSuccess || splits == 1) return e;
  int64_t blocks = cdiv(I * J, 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)blocks), dim3(256), 0, s, part, splits, I, J,
                     C, epi);
  return hipGetLastError();
}

}  // namespace brq
