// gemm.hip -- W8A8 GEMMs on gfx950 matrix cores (Open-1B report §3.2 "int8
// computation": int8 x int8 products accumulated in int32, then dequantised).
//
// Every GEMM of the layer is C[i][j] = epi(sum_k A[i][k] * B[j][k]) with both
// operands contiguous along the contraction (forward: q_x, q_w; dX: q_g,
// q_w^T; dW: the token-contiguous rotated codes q_v^T, q_u^T).  The int32
// sum is exact -- 128*128*K < 2^31 for K <= 131071 -- so tile shape, MFMA
// shape, split-K and launch order cannot change a bit of it; only the
// dequantisation epilogue is floating point:
//     out = fl(fl(acc) * c_j)   one int->fp32 conversion (round to nearest
//                               even) and one multiply, no FMA (the flush
//                               of the product can never act: see dequant).
#include "device.hpp"
#include "internal.hpp"

namespace brq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Epi {
  int kind;
  const float* s0;
  const float* s1;
  const float* s2;
  int per_row;
  float inv_b;
  int out_bf16;  // outputs rounded to bf16 (nearest even) instead of fp32
  // Column scale c_j, computed in the order the definitions give.
  __device__ __forceinline__ float scale(int64_t j) const {
    if (kind == EPI_FWD) return fmul(flush(s0[0]), flush(per_row ? s1[j] : s1[0]));
    if (kind == EPI_SCALAR) return flush(s0[0]);
    return fmul(fmul(fmul(flush(s0[0]), flush(s1[0])), flush(s2[0])), inv_b);
  }
};

// fl(fl(acc) * c) without an explicit flush: every column scale c is
// itself flushed (0 or normal), and a nonzero int32 sum converts to a
// binary32 of magnitude at least 1, so the exact product is 0 or at least
// |c| >= 2^-126 and its rounding is 0 or normal -- the flush of the
// definition never changes it.
__device__ __forceinline__ float dequant(int acc, float c) { return (float)acc * c; }

// One output element: the fp32 value, or its bf16 rounding.
__device__ __forceinline__ void put_out(float* C, int64_t idx, float v, bool bf16) {
  if (bf16) reinterpret_cast<uint16_t*>(C)[idx] = (uint16_t)f32_to_bf16(v);
  else C[idx] = v;
}

// XCD-aware tile order.  Work-group p runs on XCD p % 8 (round-robin
// dispatch), so when the tile count is a multiple of 8 the linear index is
// permuted to give each XCD a contiguous range; inside a range, groups of 8
// tile rows are swept column by column, so concurrently running tiles share
// operand rows in that XCD's L2.
__device__ __forceinline__ void tile_grouped(uint32_t p, uint32_t gm, uint32_t gn, int64_t& bm,
                                             int64_t& bn) {
  const uint32_t group = 8 * gn;
  const uint32_t g = p / group, in = p - g * group;
  const uint32_t first_m = g * 8;
  const uint32_t gsz = (gm - first_m) < 8 ? (gm - first_m) : 8;
  const uint32_t n = in / gsz;
  bm = first_m + (in - n * gsz);
  bn = n;
}
__device__ __forceinline__ void tile_of(uint32_t p, uint32_t gm, uint32_t gn, int64_t& bm,
                                        int64_t& bn) {
  // tile counts fit 32 bits (the host rejects larger launches), so the
  // index arithmetic is unsigned 32-bit
  const uint32_t total = gm * gn;
  if ((total & 7) == 0) p = (p & 7) * (total >> 3) + (p >> 3);
  tile_grouped(p, gm, gn, bm, bn);
}

// Tile and contraction slice z of a work-group of a (tiles, 1, slices)
// grid.  Work-groups go to the XCDs round-robin in launch order (x fastest,
// then z), so with one slice tile_of applies.  With several, the (tile,
// slice) units are renumbered the same way over the whole grid: XCD x runs
// a contiguous range of them, i.e. one slice's block of neighbouring tiles
// (sharing operand panels in that XCD's L2) instead of every slice of a few
// tiles (whose contraction ranges share nothing).
__device__ __forceinline__ void unit_of(uint32_t gm, uint32_t gn, int64_t& bm, int64_t& bn,
                                        int64_t& z) {
  if (gridDim.z == 1) {
    tile_of(blockIdx.x, gm, gn, bm, bn);
    z = 0;
    return;
  }
  const uint32_t tiles = gm * gn, units = tiles * gridDim.z;
  uint32_t p = blockIdx.x + gridDim.x * blockIdx.z;
  if ((units & 7) == 0) p = (p & 7) * (units >> 3) + (p >> 3);
  const uint32_t zz = p / tiles;
  tile_grouped(p - zz * tiles, gm, gn, bm, bn);
  z = zz;
}

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
  put_out(C, i * J + j, dequant(acc, epi.scale(j)), epi.out_bf16);
}

// --------------------------------------------------------------------------
// MFMA kernel.  Block tile BM x BN, contraction step BK bytes (64 or 128),
// WGM x WGN waves, each wave a (BM/WGM) x (BN/WGN) tile of 16x16
// v_mfma_i32_16x16x64_i8 blocks.
//
// LDS holds each operand tile row-major [rows][BK bytes] in 16-byte chunks,
// chunk index XOR-ed with a row hash chosen so that the rows one MFMA
// operand read touches (16 consecutive rows, one chunk each) fall in
// distinct bank groups whether the hardware serves 8 or 16 lanes of a
// 128-bit read per cycle.  Two LDS stages: while the waves multiply out of
// one stage, the next tile's global loads are in flight in registers and
// land in the other stage; one barrier per step.
//
// MFMA operand layout (16x16x64, int8): lane l supplies 16 consecutive
// contraction bytes, k-group l>>4, of row (A) or column (B) l&15; both
// operands use the same (lane, byte) -> k map, so the product sums all 64
// contraction terms.  Result: lane l holds rows 4*(l>>4)+r, column l&15.
// --------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int lds_swz(int row) {
  return BK / 16 == 8 ? ((row ^ (row >> 3)) & 7) : (((row >> 1) ^ (row >> 2)) & 3);
}
template <int BK>
__device__ __forceinline__ int lds_off(int row, int kc) {
  return row * BK + ((kc ^ lds_swz<BK>(row)) << 4);
}

template <int BM, int BN, int WGM, int WGN, int BK>
__global__ __launch_bounds__(WGM* WGN * 64) void k_gemm_mfma(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t I, int64_t J,
    int64_t Kc, float* __restrict__ C, int* __restrict__ Cpart, int ktiles_per_split, Epi epi) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int CH = BK / 16;  // 16-byte chunks per operand row
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int LA = BM * BK / 16 / NT, LB = BN * BK / 16 / NT;
  static_assert(LA * NT * 16 == BM * BK && LB * NT * 16 == BN * BK, "tile/threads");
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const int64_t gm = (I + BM - 1) / BM, gn = (J + BN - 1) / BN;
  int64_t bm, bn, zs;
  unit_of((uint32_t)gm, (uint32_t)gn, bm, bn, zs);
  const int64_t row0 = bm * BM, col0 = bn * BN;

  const int64_t nk_total = (Kc + BK - 1) / BK;
  const int64_t kt0 = zs * ktiles_per_split;
  int64_t kt1 = kt0 + ktiles_per_split;
  if (kt1 > nk_total) kt1 = nk_total;

  u32x4 ra[LA], rb[LB];
  auto gload = [&](int64_t kt) {
    const int64_t k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = t + NT * i, r = c / CH, kc = c % CH;
      const int64_t gr = row0 + r, gk = k0 + kc * 16;
      ra[i] = (gr < I && gk < Kc) ? ld16(A + gr * Kc + gk) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int c = t + NT * i, r = c / CH, kc = c % CH;
      const int64_t gr = col0 + r, gk = k0 + kc * 16;
      rb[i] = (gr < J && gk < Kc) ? ld16(B + gr * Kc + gk) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int c = t + NT * i;
      st16(&As[st][lds_off<BK>(c / CH, c % CH)], ra[i]);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int c = t + NT * i;
      st16(&Bs[st][lds_off<BK>(c / CH, c % CH)], rb[i]);
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
          af[i] = *reinterpret_cast<const v4i*>(&As[st][lds_off<BK>(r, kc)]);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int r = wn * WN + j * 16 + (lane & 15);
          bf[j] = *reinterpret_cast<const v4i*>(&Bs[st][lds_off<BK>(r, kc)]);
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
        if (Cpart) Cpart[(zs * I + row) * J + col] = acc[i][j][r];
        else put_out(C, row * J + col, dequant(acc[i][j][r], c), epi.out_bf16);
      }
    }
  }
}

// --------------------------------------------------------------------------
// Deep-pipelined MFMA kernel: operand tiles go from global memory straight
// into LDS (global_load_lds_dwordx4: each lane's 16 bytes land at the
// instruction's LDS base + 16 * lane), through kStages LDS stages, with the
// loads for contraction step t + kStages - 1 issued while step t is
// multiplied -- so each load has kStages - 1 steps of MFMA work to arrive.
// BK = 64 bytes (4 chunks of 16 per operand row) through 4 stages, or
// BK = 128 (8 chunks: every load request covers a whole 128-byte line, two
// MFMA sub-steps per step) through 2 stages of 64 KiB.  The XOR-swizzled LDS
// layout of the register-staged kernel is kept: since a lane's LDS slot is
// fixed by its lane number, each lane picks the global chunk that belongs in
// its slot.  Rows past the matrix edge read a clamped (valid) row; they only
// feed output rows or columns that are never stored.  The contraction
// length must be a multiple of 64 (no partial chunks).
//
// Synchronisation per step: wait until this wave's loads of step t have
// landed (vmcnt counts only the direct-to-LDS loads issued in the loop),
// one workgroup barrier (every wave's step-t data is in LDS and every wave
// has finished reading step t - 1's stage), read step t's fragments, issue
// the first MFMA row groups, then the loads of step t + kStages - 1 into the
// freed stage, then the remaining MFMAs.  The barrier is the bare
// s_barrier: the loads are tracked by the explicit wait, not by a fence.
// --------------------------------------------------------------------------
constexpr int kStages = 4;
// MFMA row groups of a step issued before that step's loads
constexpr int kIssueAfter = 2;

// Epilogue of one output tile, staged through LDS so that every global
// store instruction writes whole rows (bf16 outputs: half rows of 512 bytes): one wave's 16-byte-per-lane store
// covers BN * 4 / 1024 rows of 1 KiB contiguous (one row for BN = 256).
// Straight from the MFMA layout (one column, four rows per lane) a store
// instruction would touch 16 rows 64 bytes each, and the output write runs
// about 2.5x slower per CU.  Per 16-row block of the tile: every wave
// writes its 16 x WN values (dequantised, or raw int32 for split-K
// partials) into the staging area -- WGM groups of 16 rows x BN words, 16-byte
// chunks XOR-swizzled by row -- barrier, then the waves of each row group
// read back whole rows and store them, barrier.  The fp32 outputs go out as
// non-temporal (streaming) stores: nothing in the kernel reads them back.
// Split-K partials (slice z) are cached: the reduction reads them.
// scale(j) gives the column scale c_j.  The caller guarantees that no wave
// still reads `stage` and that no load is in flight into it.
template <int BM, int BN, int WGM, int WGN, class Scale>
__device__ __forceinline__ void store_tile(const v4i (&acc)[BM / WGM / 16][BN / WGN / 16],
                                           int64_t row0, int64_t col0, int wave, int lane,
                                           int64_t I, int64_t J, float* __restrict__ C,
                                           int* __restrict__ Cpart, int64_t z,
                                           const Scale& scale, int8_t* stage, bool obf16) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int CPR = BN / 4;                 // 16-byte chunks per staged row
  constexpr int GROUP = 16 * BN * 4;          // bytes per row group
  constexpr int RCH = 16 * CPR / (WGN * 64);  // chunks each lane stores per block
  static_assert(CPR >= 8 && RCH * WGN * 64 == 16 * CPR && RCH % 2 == 0, "staging layout");
  const int wm = wave / WGN, wn = wave % WGN;
  int8_t* grp = stage + wm * GROUP;
  const int rq = 4 * (lane >> 4);  // first of the lane's 4 rows in a block
  const int cc = wn * WN + (lane & 15);  // the lane's column in j-block 0
  float cj[TJ];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t col = col0 + cc + j * 16;
    cj[j] = (!Cpart && col < J) ? scale(col) : 0.0f;
  }
  auto word = [&](int r, int c) {  // byte offset of staged word (r, c)
    return (r * CPR + ((c >> 2) ^ (r & 7))) * 16 + (c & 3) * 4;
  };
#pragma unroll  // fully: acc must stay in registers
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int v = acc[i][j][r];
        const int bits = Cpart ? v : __float_as_int(dequant(v, cj[j]));
        *reinterpret_cast<int*>(grp + word(rq + r, cc + j * 16)) = bits;
      }
    }
    __syncthreads();
    if (obf16 && !Cpart) {
      // bf16: each lane takes two adjacent chunks (8 columns) and stores 16
      // bytes, so a store instruction still writes whole 512-byte rows
#pragma unroll
      for (int k = 0; k < RCH / 2; ++k) {
        const int pr = (k * WGN + wn) * 64 + lane;  // chunk pair of the group
        const int r = pr / (CPR / 2), c8 = pr % (CPR / 2);
        const v4i a = *reinterpret_cast<const v4i*>(grp + (r * CPR + ((2 * c8) ^ (r & 7))) * 16);
        const v4i b =
            *reinterpret_cast<const v4i*>(grp + (r * CPR + ((2 * c8 + 1) ^ (r & 7))) * 16);
        const int64_t row = row0 + wm * WM + i * 16 + r;
        const int64_t col = col0 + c8 * 8;
        if (row >= I || col >= J) continue;
        uint16_t* dst = reinterpret_cast<uint16_t*>(C) + row * J + col;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          w[e] = f32_to_bf16(__int_as_float(a[2 * e])) |
                 (f32_to_bf16(__int_as_float(a[2 * e + 1])) << 16);
          w[2 + e] = f32_to_bf16(__int_as_float(b[2 * e])) |
                     (f32_to_bf16(__int_as_float(b[2 * e + 1])) << 16);
        }
        if (col + 8 <= J && (J & 7) == 0) {
          __builtin_nontemporal_store(v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]},
                                      reinterpret_cast<v4i*>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < J) dst[e] = (uint16_t)((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        }
      }
      __syncthreads();
      continue;
    }
#pragma unroll
    for (int k = 0; k < RCH; ++k) {
      const int ch = (k * WGN + wn) * 64 + lane;  // chunk of the group
      const int r = ch / CPR, c4 = ch % CPR;
      const v4i v = *reinterpret_cast<const v4i*>(grp + (r * CPR + (c4 ^ (r & 7))) * 16);
      const int64_t row = row0 + wm * WM + i * 16 + r;
      const int64_t col = col0 + c4 * 4;
      if (row >= I || col >= J) continue;
      const bool full = col + 4 <= J && (J & 3) == 0;
      if (Cpart) {
        int* dst = Cpart + (z * I + row) * J + col;
        if (full) {
          *reinterpret_cast<v4i*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < J) dst[e] = v[e];
        }
      } else {
        float* dst = C + row * J + col;
        if (full) {
          __builtin_nontemporal_store(
              f32x4{__int_as_float(v[0]), __int_as_float(v[1]), __int_as_float(v[2]),
                    __int_as_float(v[3])},
              reinterpret_cast<f32x4*>(dst));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < J) dst[e] = __int_as_float(v[e]);
        }
      }
    }
    __syncthreads();
  }
}

// Epilogue of a tile wholly inside an fp32 output, or inside a split-K
// slice of int32 partials (Cpart != nullptr, slice z), staged per wave
// instead of per row group: each wave writes its 16 x WN block into a
// private LDS area (16 * WN * 4 bytes; all waves together take the same
// space as the per-group staging) and reads it back as 16-byte chunks, so
// one store instruction writes 64 * 16 bytes in whole rows of WN * 4
// contiguous bytes (256 bytes, two 128-byte lines, for WN = 64).  A wave's own LDS writes and reads
// execute in order, so no work-group barrier is needed.  The 16-byte
// chunk index is XOR-ed with row bit 2: the four row groups of a 32-bit
// write then cover all 32 banks twice, and the 8 lanes of a 128-bit read
// cycle hit 8 different chunks.  Offsets and global addresses are
// computed once per tile.
template <int BM, int BN, int WGM, int WGN, class Scale>
__device__ __forceinline__ void store_tile_full(const v4i (&acc)[BM / WGM / 16][BN / WGN / 16],
                                                int64_t row0, int64_t col0, int wave, int lane,
                                                int64_t I, int64_t J, float* __restrict__ C,
                                                int* __restrict__ Cpart, int64_t z,
                                                const Scale& scale, int8_t* stage) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int CPW = WN / 4;     // 16-byte chunks per staged row
  constexpr int KR = 16 * CPW / 64;  // chunks each lane reads back per block
  static_assert(CPW >= 8 && CPW <= 64 && KR * 64 == 16 * CPW, "staging layout");
  const int wm = wave / WGN, wn = wave % WGN;
  int8_t* own = stage + wave * (16 * WN * 4);
  const int rq = 4 * (lane >> 4);
  const int lcol = lane & 15;  // the lane's column in each 16-column block
  float cj[TJ];
  int woff[TJ][4];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    cj[j] = Cpart ? 0.0f : scale(col0 + wn * WN + lcol + j * 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = rq + r, c = lcol + j * 16;
      woff[j][r] = row * (WN * 4) + (((c >> 2) ^ (((row >> 2) & 1) << 2)) << 4) + (c & 3) * 4;
    }
  }
  // read-back: chunk x = lane % CPW of rows (64 / CPW) k + lane / CPW
  int roff[KR];
  int64_t eoff[KR];
  const int64_t zbase = Cpart ? z * I * J : 0;
#pragma unroll
  for (int k = 0; k < KR; ++k) {
    const int row = (64 / CPW) * k + lane / CPW, x = lane % CPW;
    roff[k] = row * (WN * 4) + ((x ^ (((row >> 2) & 1) << 2)) << 4);
    eoff[k] = zbase + (row0 + wm * WM + row) * J + col0 + wn * WN + x * 4;
  }
#pragma unroll  // fully: acc must stay in registers
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<int*>(own + woff[j][r]) =
            Cpart ? acc[i][j][r] : __float_as_int(dequant(acc[i][j][r], cj[j]));
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const v4i v = *reinterpret_cast<const v4i*>(own + roff[k]);
      const int64_t e = eoff[k] + (int64_t)i * 16 * J;
      // partials are cached (the reduction reads them); outputs stream
      if (Cpart)
        *reinterpret_cast<v4i*>(Cpart + e) = v;
      else
        __builtin_nontemporal_store(f32x4{__int_as_float(v[0]), __int_as_float(v[1]),
                                          __int_as_float(v[2]), __int_as_float(v[3])},
                                    reinterpret_cast<f32x4*>(C + e));
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int BK = 64, int NS = kStages>
__global__ __launch_bounds__(WGM* WGN * 64) void k_gemm_dma(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t I, int64_t J,
    int64_t Kc, float* __restrict__ C, int* __restrict__ Cpart, int ktiles_per_split, Epi epi) {
  static_assert((BK == 64 && NS >= 2) || (BK == 128 && NS == 2), "step and stages");
  constexpr int CH = BK / 16;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int DA = BM * CH / 64 / NW, DB = BN * CH / 64 / NW;  // loads per wave per step
  constexpr int L = DA + DB;
  static_assert(DA * 64 * NW == BM * CH && DB * 64 * NW == BN * CH, "tile/waves");
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(WGM * 16 * BN * 4 <= NS * STAGE, "epilogue staging fits the stages");
  __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const int64_t gm = (I + BM - 1) / BM, gn = (J + BN - 1) / BN;
  int64_t bm, bn, zs;
  unit_of((uint32_t)gm, (uint32_t)gn, bm, bn, zs);
  const int64_t row0 = bm * BM, col0 = bn * BN;

  const int64_t nk_total = Kc / BK;
  const int64_t kt0 = zs * ktiles_per_split;
  int64_t kt1 = kt0 + ktiles_per_split;
  if (kt1 > nk_total) kt1 = nk_total;
  const int64_t nk = kt1 > kt0 ? kt1 - kt0 : 0;

  // per-lane source of each direct-to-LDS load: slot sigma of the stage's
  // A (then B) region holds row sigma / 4, chunk (sigma % 4) ^ f(row)
  const int8_t* srcA[DA];
  const int8_t* srcB[DB];
#pragma unroll
  for (int i = 0; i < DA; ++i) {
    const int sg = (wave * DA + i) * 64 + lane, r = sg / CH;
    const int f = lds_swz<BK>(r);
    int64_t gr = row0 + r;
    gr = gr < I ? gr : I - 1;
    srcA[i] = A + gr * Kc + (int64_t)(((sg % CH) ^ f) * 16) + kt0 * BK;
  }
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int sg = (wave * DB + i) * 64 + lane, r = sg / CH;
    const int f = lds_swz<BK>(r);
    int64_t gr = col0 + r;
    gr = gr < J ? gr : J - 1;
    srcB[i] = B + gr * Kc + (int64_t)(((sg % CH) ^ f) * 16) + kt0 * BK;
  }
  auto issue = [&](int64_t it) {
    int8_t* st = smem + (it % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < DA; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcA[i] + it * BK),
          (__attribute__((address_space(3))) void*)(st + (wave * DA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < DB; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcB[i] + it * BK),
          (__attribute__((address_space(3))) void*)(st + BM * BK + (wave * DB + i) * 1024), 16,
          0, 0);
  };

  v4i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s);

  const int kc = lane >> 4;
#pragma unroll 1
  for (int64_t it = 0; it < nk; ++it) {
    // loads still allowed in flight: those of the (up to NS - 2) later
    // steps already issued
    const int64_t later = nk - 1 - it;
    if (NS >= 4 && later >= 2) wait_vmcnt<(NS >= 4 ? 2 : 0) * L>();
    else if (NS >= 3 && later >= 1) wait_vmcnt<(NS >= 3 ? 1 : 0) * L>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const int8_t* st = smem + (it % NS) * STAGE;
    if constexpr (BK == 64) {
      v4i af[TI], bf[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wm * WM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const v4i*>(st + lds_off<BK>(r, kc));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = wn * WN + j * 16 + (lane & 15);
        bf[j] = *reinterpret_cast<const v4i*>(st + BM * BK + lds_off<BK>(r, kc));
      }
      constexpr int IA = kIssueAfter < TI ? kIssueAfter : TI;
#pragma unroll
      for (int i = 0; i < IA; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (it + NS - 1 < nk) issue(it + NS - 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = IA; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      asm volatile("" ::: "memory");
    } else {
      // two MFMA sub-steps per 128-byte step; the next loads go out after the
      // first one's leading row groups
#pragma unroll
      for (int kh = 0; kh < BK / 64; ++kh) {
        v4i af[TI], bf[TJ];
#pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int r = wm * WM + i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const v4i*>(st + lds_off<BK>(r, 4 * kh + kc));
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const int r = wn * WN + j * 16 + (lane & 15);
          bf[j] = *reinterpret_cast<const v4i*>(st + BM * BK + lds_off<BK>(r, 4 * kh + kc));
        }
        constexpr int IA = kIssueAfter < TI ? kIssueAfter : TI;
#pragma unroll
        for (int i = 0; i < IA; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (kh == 0 && it + NS - 1 < nk) issue(it + NS - 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = IA; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        asm volatile("" ::: "memory");
      }
    }
  }

  // every load has landed (the last step waited for all); the barrier
  // frees the stages for the epilogue
  __syncthreads();
  if ((Cpart || !epi.out_bf16) && row0 + BM <= I && col0 + BN <= J && (J & 3) == 0)
    store_tile_full<BM, BN, WGM, WGN>(acc, row0, col0, wave, lane, I, J, C, Cpart, zs,
                                      [&](int64_t j) { return epi.scale(j); }, smem);
  else
    store_tile<BM, BN, WGM, WGN>(acc, row0, col0, wave, lane, I, J, C, Cpart, zs,
                                 [&](int64_t j) { return epi.scale(j); }, smem, epi.out_bf16);
}

// --------------------------------------------------------------------------
// Persistent form of the direct-to-LDS kernel.  One work-group per CU walks
// work units u = blockIdx.x, blockIdx.x + gridDim.x, ... (a unit is one
// output tile of one contraction slice: u = slice * tiles + tile), and the
// load pipeline runs across unit boundaries: the loads of the next unit's
// first kStages - 1 steps are issued during the last steps of the current
// unit and land while its epilogue runs, so no tile starts on a cold
// pipeline.  Unit u runs on XCD u % 8 when the grid is a multiple of 8, as
// tile u does in the one-tile-per-group launch, so the same tile order
// applies.
//
// Every unit needs at least kStages contraction steps.  The issue cursor
// runs kStages - 1 steps ahead, so it then enters unit u + 2 (and loads
// that unit's column scales into the buffer of unit u's parity) only after
// unit u's epilogue has read them.
//
// The wait before step t allows the loads of the steps already issued after
// t to stay in flight.  Any other memory operation still outstanding (the
// previous tile's stores) only makes that wait stricter: loads complete in
// order among themselves, so step t's loads cannot be pending while fewer
// ops than the later steps' loads are.
// --------------------------------------------------------------------------
template <int L, int MAXL>
__device__ __forceinline__ void wait_later(int64_t later) {
  if constexpr (MAXL == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<MAXL * L>();
    else wait_later<L, MAXL - 1>(later);
  }
}

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(WGM* WGN * 64) void k_gemm_stream(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, int64_t I, int64_t J,
    int64_t Kc, float* __restrict__ C, int* __restrict__ Cpart, int ktiles_per_split,
    int splits, Epi epi) {
  constexpr int BK = 64, CH = BK / 16;
  constexpr int NW = WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int TI = WM / 16, TJ = WN / 16;
  constexpr int DA = BM * CH / 64 / NW, DB = BN * CH / 64 / NW;  // loads per wave per step
  constexpr int L = DA + DB;
  static_assert(DA * 64 * NW == BM * CH && DB * 64 * NW == BN * CH, "tile/waves");
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(BN % 64 == 0 && BN / 64 <= NW, "one scale load per wave");
  static_assert(kIssueAfter <= TI, "issue point inside the MFMA rows");
  static_assert(WGM * 16 * BN * 4 <= STAGE, "epilogue staging fits one stage");
  __shared__ __attribute__((aligned(1024))) int8_t smem[kStages * STAGE];
  __shared__ __attribute__((aligned(16))) float cs[2][BN];  // per-unit column scales

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t gm = (I + BM - 1) / BM, gn = (J + BN - 1) / BN;
  const int64_t tiles = gm * gn, units = tiles * splits;
  // Column scales: a per-output-channel forward scale s1[j] travels with
  // the operand loads (one direct-to-LDS load per unit into cs[unit
  // parity], issued just before the unit's first stage, so it has landed
  // once that stage has); every other scale is uniform and read here, before
  // any load is in flight.
  const bool col_scales = !Cpart && epi.kind == EPI_FWD && epi.per_row;
  const float c_uni = Cpart ? 0.0f : col_scales ? flush(epi.s0[0]) : epi.scale(0);
  const int64_t nk_total = Kc / BK;
  const int64_t G = gridDim.x;

  struct Unit {
    int64_t row0, col0, kt0, nk;
  };
  auto unit_at = [&](int64_t u) {
    Unit w;
    const uint32_t z = (uint32_t)u / (uint32_t)tiles;
    int64_t bm, bn;
    tile_of((uint32_t)u - z * (uint32_t)tiles, (uint32_t)gm, (uint32_t)gn, bm, bn);
    w.row0 = bm * BM;
    w.col0 = bn * BN;
    w.kt0 = z * ktiles_per_split;
    int64_t kt1 = w.kt0 + ktiles_per_split;
    if (kt1 > nk_total) kt1 = nk_total;
    w.nk = kt1 > w.kt0 ? kt1 - w.kt0 : 0;
    return w;
  };

  // per-lane part of each direct-to-LDS load: slot sigma of the stage's A
  // (then B) region holds row sigma / 4, chunk (sigma % 4) ^ f(row)
  int rowA[DA], offA[DA], rowB[DB], offB[DB];
#pragma unroll
  for (int i = 0; i < DA; ++i) {
    const int sg = (wave * DA + i) * 64 + lane, r = sg / CH;
    rowA[i] = r;
    offA[i] = ((sg % CH) ^ (((r >> 1) ^ (r >> 2)) & 3)) * 16;
  }
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    const int sg = (wave * DB + i) * 64 + lane, r = sg / CH;
    rowB[i] = r;
    offB[i] = ((sg % CH) ^ (((r >> 1) ^ (r >> 2)) & 3)) * 16;
  }

  // issue cursor: unit ui, its step iit of inks, ring slot islot
  const int8_t* srcA[DA];
  const int8_t* srcB[DB];
  int64_t ui = blockIdx.x, iit = 0, inks = 0, issued = 0;
  int islot = 0;
  uint32_t iord = 0;  // ordinal of unit ui in this work-group's sequence
  auto seek = [&]() {  // first unit at or after ui with contraction steps
    for (; ui < units; ui += G, ++iord) {
      const Unit w = unit_at(ui);
      if (w.nk == 0) continue;
      inks = w.nk;
      if (col_scales && wave < BN / 64) {
        int64_t c = w.col0 + wave * 64 + lane;
        c = c < J ? c : J - 1;
        __builtin_amdgcn_global_load_lds(
            (const void*)(epi.s1 + c),
            (__attribute__((address_space(3))) void*)(&cs[iord & 1][wave * 64]),
            4, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < DA; ++i) {
        int64_t gr = w.row0 + rowA[i];
        gr = gr < I ? gr : I - 1;
        srcA[i] = A + gr * Kc + offA[i] + w.kt0 * BK;
      }
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        int64_t gr = w.col0 + rowB[i];
        gr = gr < J ? gr : J - 1;
        srcB[i] = B + gr * Kc + offB[i] + w.kt0 * BK;
      }
      return;
    }
  };
  auto issue_next = [&]() {
    if (ui >= units) return;
    int8_t* st = smem + islot * STAGE;
#pragma unroll
    for (int i = 0; i < DA; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcA[i] + iit * BK),
          (__attribute__((address_space(3))) void*)(st + (wave * DA + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < DB; ++i)
      __builtin_amdgcn_global_load_lds(
          (const void*)(srcB[i] + iit * BK),
          (__attribute__((address_space(3))) void*)(st + BM * BK + (wave * DB + i) * 1024), 16,
          0, 0);
    islot = islot == kStages - 1 ? 0 : islot + 1;
    ++issued;
    if (++iit == inks) {
      iit = 0;
      ui += G;
      ++iord;
      seek();
    }
  };

  v4i acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  seek();
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue_next();

  const int kc = lane >> 4;
  int cslot = 0;
  int64_t computed = 0;
  uint32_t cord = 0;  // ordinal of unit uc
  // store instructions this wave issued in the previous unit's epilogue
  // that certainly follow the loads of this unit's first kStages - 1 steps
  // (loads and stores complete in issue order, so the first kStages - 1
  // waits of a unit may leave them in flight); 0 where not certain
  constexpr int kStoreInstr = BM / WGM / 16 * (16 * (BN / 4) / (WGN * 64));
  int stores_prev = 0;
#pragma unroll 1
  for (int64_t uc = blockIdx.x; uc < units; uc += G, ++cord) {
    const Unit w = unit_at(uc);
#pragma unroll 1
    for (int64_t it = 0; it < w.nk; ++it) {
      if (it < kStages - 1 && stores_prev > 0)
        wait_vmcnt_upto<(kStages - 2) * L + kStoreInstr>((int)(issued - computed - 1) * L +
                                                          stores_prev);
      else
        wait_later<L, kStages - 2>(issued - computed - 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" ::: "memory");
      const int8_t* st = smem + cslot * STAGE;
      v4i af[TI], bf[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wm * WM + i * 16 + (lane & 15);
        af[i] = *reinterpret_cast<const v4i*>(st + lds_off<BK>(r, kc));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = wn * WN + j * 16 + (lane & 15);
        bf[j] = *reinterpret_cast<const v4i*>(st + BM * BK + lds_off<BK>(r, kc));
      }
      // the next loads go out after the fragment reads and the first MFMA
      // row group: issued right after the barrier, all waves' loads queue
      // at once and hold up the reads and MFMAs behind them
#pragma unroll
      for (int i = 0; i < kIssueAfter; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      issue_next();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = kIssueAfter; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      asm volatile("" ::: "memory");
      cslot = cslot == kStages - 1 ? 0 : cslot + 1;
      ++computed;
    }
    const float* cu = cs[cord & 1];
    // stage through the slot the last step consumed: the loads in flight
    // target the other kStages - 1 slots, and the next load into this one
    // is issued after the next step's barrier
    const int last = cslot == 0 ? kStages - 1 : cslot - 1;
    __syncthreads();  // every wave has read its last fragments
    const auto unit_scale = [&](int64_t j) {
      return col_scales ? fmul(c_uni, flush(cu[j - w.col0])) : c_uni;
    };
    if ((Cpart || !epi.out_bf16) && w.row0 + BM <= I && w.col0 + BN <= J && (J & 3) == 0)
      store_tile_full<BM, BN, WGM, WGN>(acc, w.row0, w.col0, wave, lane, I, J, C, Cpart,
                                        (uint32_t)uc / (uint32_t)tiles, unit_scale,
                                        smem + last * STAGE);
    else
      store_tile<BM, BN, WGM, WGN>(acc, w.row0, w.col0, wave, lane, I, J, C, Cpart,
                                   (uint32_t)uc / (uint32_t)tiles, unit_scale,
                                   smem + last * STAGE, epi.out_bf16);
    // a tile wholly inside the output, with rows a multiple of the store
    // width: every lane takes the one-instruction store of each chunk
    {
      const bool b16 = epi.out_bf16 && !Cpart;
      const bool whole = w.row0 + BM <= I && w.col0 + BN <= J && (J % (b16 ? 8 : 4)) == 0;
      stores_prev = whole ? (b16 ? kStoreInstr / 2 : kStoreInstr) : 0;
    }
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  }
}

// Sum of the split-K partials in split order (exact in int32), then the
// same epilogue.  Thread x of the grid owns 4 consecutive columns (J a
// multiple of 4: 16-byte partial loads and fp32 stores) or one column, so
// its column scales are formed once; rows go y, y + gridDim.y, ...
__global__ __launch_bounds__(256) void k_splitk_reduce(const int* __restrict__ Cpart, int splits,
                                                       int64_t I, int64_t J, float* __restrict__ C,
                                                       Epi epi) {
  const int64_t n = I * J;
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if ((J & 3) == 0) {
    const int64_t j = 4 * x;
    if (j >= J) return;
    float c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = epi.scale(j + k);
    for (int64_t i = blockIdx.y; i < I; i += gridDim.y) {
      const int64_t e = i * J + j;
      v4i acc = {0, 0, 0, 0};
      for (int z = 0; z < splits; ++z) acc += *reinterpret_cast<const v4i*>(Cpart + z * n + e);
      if (epi.out_bf16) {
#pragma unroll
        for (int k = 0; k < 4; ++k) put_out(C, e + k, dequant(acc[k], c[k]), true);
      } else {
        *reinterpret_cast<f32x4*>(C + e) = f32x4{dequant(acc[0], c[0]), dequant(acc[1], c[1]),
                                                 dequant(acc[2], c[2]), dequant(acc[3], c[3])};
      }
    }
  } else {
    const int64_t j = x;
    if (j >= J) return;
    const float c = epi.scale(j);
    for (int64_t i = blockIdx.y; i < I; i += gridDim.y) {
      const int64_t e = i * J + j;
      int acc = 0;
      for (int z = 0; z < splits; ++z) acc += Cpart[z * n + e];
      put_out(C, e, dequant(acc, c), epi.out_bf16);
    }
  }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch plan: the tune's kernel and split-K when given, else by shape --
// the deep-pipelined 256x256 kernel whenever the contraction is a multiple
// of 64 bytes, persistent when there are more tiles than CUs and each
// tile's contraction is short, with the contraction split so that tiles x
// splits reaches about one work-group per CU when the output has few
// tiles.  None of this
// changes a result bit: the int32 sums are exact in any grouping.
// Work-groups the persistent kernel keeps resident: one per CU (its LDS
// stages take most of a CU's LDS).
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

struct Plan {
  int kern;
  int splits;
};

static Plan plan_of(int64_t I, int64_t J, int64_t Kc, const brq_tune* t) {
  Plan p{2, 1};
  const int tk = t ? t->gemm_kernel : 0;
  const int ts = t ? t->split_k : 0;
  if (tk) {
    p.kern = tk;
  } else if (Kc % 64 == 0) {
    p.kern = 10;
  }
  if (ts) {
    p.splits = (ts == 2 || ts == 4 || ts == 8 || ts == 16) ? ts : 1;
  } else if (!tk && p.kern == 10) {
    const int64_t tiles = cdiv(I, 256) * cdiv(J, 256);
    int s = 1;
    while (s < 16 && tiles * s < 256 && Kc / 64 / (2 * s) >= 32) s *= 2;
    p.splits = s;
    // persistent when each CU gets several tiles of a short contraction
    // (a tile start costs the most there); long ones run as well or
    // better one tile per group
    const int64_t steps = Kc / 64 / s;
    if (tiles * s > cu_count() && steps >= kStages && steps < 64 && (Kc / 64) % s == 0)
      p.kern = 13;
    // one tile per work-group over a long contraction (the weight-gradient
    // GEMMs of the wide linears): 128-byte steps, whole-line load requests
    else if (s == 1 && tiles <= cu_count() && Kc >= 8192 && Kc % 128 == 0)
      p.kern = 14;
  }
  if (p.kern == 1) p.splits = 1;
  return p;
}

size_t gemm_ws(int64_t I, int64_t J, int64_t Kc, const brq_tune* t) {
  const Plan p = plan_of(I, J, Kc, t);
  if (p.splits == 1) return 0;
  return align256((size_t)p.splits * (size_t)I * (size_t)J * sizeof(int));
}

template <int BM, int BN, int WGM, int WGN, int BK>
static hipError_t launch_mfma(const int8_t* A, const int8_t* B, int64_t I, int64_t J, int64_t Kc,
                              float* C, int* Cpart, int splits, Epi epi, hipStream_t s) {
  const int64_t tiles = cdiv(I, BM) * cdiv(J, BN);
  const int64_t nk = cdiv(Kc, BK);
  const int kps = (int)cdiv(nk, splits);
  dim3 g((unsigned)tiles, 1, (unsigned)splits), b(WGM * WGN * 64);
  hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN, BK>), g, b, 0, s, A, B, I, J, Kc, C, Cpart, kps,
                     epi);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int BK = 64, int NS = kStages>
static hipError_t launch_dma(const int8_t* A, const int8_t* B, int64_t I, int64_t J, int64_t Kc,
                             float* C, int* Cpart, int splits, Epi epi, hipStream_t s) {
  const int64_t tiles = cdiv(I, BM) * cdiv(J, BN);
  const int64_t nk = Kc / BK;
  const int kps = (int)cdiv(nk, splits);
  dim3 g((unsigned)tiles, 1, (unsigned)splits), b(WGM * WGN * 64);
  hipLaunchKernelGGL((k_gemm_dma<BM, BN, WGM, WGN, BK, NS>), g, b, 0, s, A, B, I, J, Kc, C, Cpart,
                     kps, epi);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_stream(const int8_t* A, const int8_t* B, int64_t I, int64_t J,
                                int64_t Kc, float* C, int* Cpart, int splits, Epi epi,
                                hipStream_t s) {
  const int64_t units = cdiv(I, BM) * cdiv(J, BN) * splits;
  const int64_t nk = Kc / 64;
  const int kps = (int)cdiv(nk, splits);
  int64_t grid = cu_count();
  if (grid > units) grid = units;
  hipLaunchKernelGGL((k_gemm_stream<BM, BN, WGM, WGN>), dim3((unsigned)grid), dim3(WGM * WGN * 64),
                     0, s, A, B, I, J, Kc, C, Cpart, kps, splits, epi);
  return hipGetLastError();
}

hipError_t gemm_i8(const int8_t* A, const int8_t* B, int64_t I, int64_t J, int64_t Kc, float* C,
                   const EpiArgs& ea, void* ws, size_t ws_bytes, const brq_tune* t,
                   hipStream_t s) {
  Epi epi{ea.kind, ea.s0, ea.s1, ea.s2, ea.per_row, ea.inv_b, ea.out_bf16};
  if (I == 0 || J == 0) return hipSuccess;
  // tile indices are unsigned 32-bit: at most 2^31 work units of the
  // smallest tile (128 x 128) times the largest split
  if (cdiv(I, 128) * cdiv(J, 128) * 16 > (int64_t)INT32_MAX) return hipErrorInvalidValue;
  const Plan pl = plan_of(I, J, Kc, t);
  int kern = pl.kern;
  if (kern == 1) {
    dim3 g((unsigned)cdiv(J, 64), (unsigned)cdiv(I, 4)), b(256);
    hipLaunchKernelGGL(k_gemm_ref, g, b, 0, s, A, B, I, J, Kc, C, epi);
    return hipGetLastError();
  }
  const int splits = pl.splits;
  int* part = nullptr;
  if (splits > 1) {
    if (ws_bytes < gemm_ws(I, J, Kc, t)) return hipErrorInvalidValue;
    part = (int*)ws;
  }
  hipError_t e;
  // the direct-to-LDS kernels need whole 64-byte (kernel 14: 128-byte)
  // contraction chunks
  if (kern == 14 && Kc % 128) kern = 10;
  if (kern >= 9 && kern <= 13 && Kc % 64) kern = 2;
  switch (kern) {
    case 9: e = launch_dma<256, 256, 2, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 10: e = launch_dma<256, 256, 2, 4>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 11: e = launch_dma<128, 256, 2, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 12: e = launch_dma<128, 128, 2, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 14: e = launch_dma<256, 256, 2, 4, 128, 2>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 13:
      // every unit must hold at least kStages contraction steps
      if (Kc / 64 / splits >= kStages && (Kc / 64) % splits == 0)
        e = launch_stream<256, 256, 2, 4>(A, B, I, J, Kc, C, part, splits, epi, s);
      else
        e = launch_dma<256, 256, 2, 4>(A, B, I, J, Kc, C, part, splits, epi, s);
      break;
    case 3: e = launch_mfma<256, 128, 2, 2, 128>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 4: e = launch_mfma<128, 256, 2, 2, 128>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 5: e = launch_mfma<256, 256, 2, 2, 64>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 6: e = launch_mfma<256, 256, 2, 2, 128>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 7: e = launch_mfma<256, 256, 2, 4, 64>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    case 8: e = launch_mfma<256, 256, 4, 2, 128>(A, B, I, J, Kc, C, part, splits, epi, s); break;
    default: e = launch_mfma<128, 128, 2, 2, 128>(A, B, I, J, Kc, C, part, splits, epi, s); break;
  }
  if (e != hipSuccess || splits == 1) return e;
  // columns across x (4 per thread when J % 4 == 0), rows across y: about
  // 2048 work-groups, each thread walking I / gridDim.y rows
  const int64_t gx = cdiv((J & 3) == 0 ? J / 4 : J, 256);
  int64_t gy = 2048 / gx;
  if (gy < 1) gy = 1;
  if (gy > I) gy = I;
  if (gy > 65535) gy = 65535;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, s, part, splits, I, J,
                     C, epi);
  return hipGetLastError();
}

}  // namespace brq
