// dy.hip -- both int8 codes of the upstream gradient dY in two passes over
// it (Open-1B report §3.2 "int8 computation": both straight-through
// gradient GEMMs run in int8, the weight-gradient one after a Walsh-Hadamard
// rotation along the contraction dimension, i.e. tokens).
//
//   q_g  = LSQ per tensor of g = fl(dY * s_w[n])        (input-gradient GEMM)
//   q_vt = LSQ per tensor of v = fp32 butterflies of dY
//          along tokens in aligned blocks, written
//          token-contiguous [N][M]                     (weight-gradient GEMM)
//
// The definitions are those of quantize_lsq with col_mul and of
// wht_quant_dy; only the data movement is fused.  Both statistics are the
// canonical pairwise tree over their leaves in row-major [M][N] order.
// Every 64 aligned leaves of a row form one node(6, .) of that tree
// (N % 64 == 0, so no run crosses a row), and the node(6) arrays, in
// row-major order of (row, column / 64), are reduced by the flat tree --
// levels 6 and up of the same tree.
//
// Tile: 128 tokens x 128 columns of bf16 per 256-thread work-group.
//   row phase:    16-byte loads (8 columns of one row per lane); the g
//                 leaves of 8 lanes (64 columns) pair up in registers and
//                 through three DPP butterfly steps; the tile lands in LDS.
//   column phase: wave w owns columns 32w .. 32w+31; lane l holds column
//                 32w + (l & 31), tokens 64 (l >> 5) .. +63.  Butterfly
//                 stages h = 1 .. 32 run in registers; stage 64 pairs lane l
//                 with lane l ^ 32, one register swap per two values, after
//                 which the halves hold tokens in the order tok_after gives.
//                 The |v| leaves go back through LDS to row order, 64 rows
//                 at a time, to form node(6) per row and 64 columns.
// The node(6) arrays are stored tile by tile (TileMap): a tile's 128 rows x
// 2 nodes are one contiguous 1 KiB run, so its node stores fill whole
// lines; the reduction reads them in the row-major order of the tree.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

constexpr int kRows = 128;                 // tokens per tile
constexpr int kCols = 128;                 // columns per tile
constexpr int kHalf = 64;                  // tokens per lane in the column phase
constexpr int kRowBytes = kCols * 2 + 16;  // padded LDS row of the bf16 tile
constexpr int kTrStride = kCols + 4;       // padded fp32 row of the |v| transpose

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row phase shared by both passes: lane t covers columns 8 (t & 15) .. +7 of
// rows (t >> 4) + 16 i, i = 0..7.  The row addresses step by 16 N from the
// first one (64-bit adds, not a 64-bit multiply per row).
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ dy, int64_t N, int64_t m0,
                                          int64_t col, int rb, u32x4 (&raw)[kRows / 16]) {
  const uint16_t* p = dy + (m0 + rb) * N + col;
  const int64_t step = 16 * N;
#pragma unroll
  for (int i = 0; i < kRows / 16; ++i) {
    raw[i] = col < N ? ld16(p) : u32x4{0, 0, 0, 0};
    p += step;
  }
}

// The lane's 8 column steps (DAZ); N % 64 == 0 and colv % 8 == 0, so the 8
// columns are all inside the matrix or all outside it.
__device__ __forceinline__ void load_steps(const float* __restrict__ sw, int64_t N, int64_t colv,
                                           float* s8) {
  if (colv < N) {
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = flush(sw[colv + e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) s8[e] = 0.0f;
  }
}

// Fast-path test, exact (the argument under column_wht): a bf16 tile whose
// nonzero values all have magnitude >= 2^-103 has only normal inputs, and
// every product with a step |s| >= 2^-23 (or 0) and every butterfly sum
// and difference is normal or zero, so each flush is the identity.  The
// test runs on 16-bit pairs: |h| - 1 wraps a zero to 0xffff, and the
// packed minimum must stay >= 0x0BFF (the pattern of 2^-103 is 0x0C00).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 tiny_min(u16x2 lo, u32x4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const u16x2 one = {1, 1};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    u16x2 h = __builtin_bit_cast(u16x2, w[k] & 0x7fff7fffu);
    lo = __builtin_elementwise_min(lo, h - one);
  }
  return lo;
}
__device__ __forceinline__ bool tiny_ok(u16x2 lo) { return lo.x >= 0x0BFFu && lo.y >= 0x0BFFu; }
// the row phase's products also need every step |s| >= 2^-23 or s = 0
__device__ __forceinline__ bool steps_ok(const float* s8) {
  bool ok = true;
#pragma unroll
  for (int e = 0; e < 8; ++e) ok = ok && (s8[e] == 0.0f || fabsf(s8[e]) >= 0x1p-23f);
  return ok;
}

// Column phase: the lane's 64 tokens of its column (DAZ), then the
// butterflies in stage order h = 1, 2, ..., b/2, each a rounded sum and
// difference (v_j, v_j+h) <- (fl(v_j + v_j+h), fl(v_j - v_j+h)).
//
// Fast path, exact: if every nonzero input of the wave has magnitude
// >= 2^-103, every input is a multiple of 2^-110 (a bf16 value of exponent e
// is a multiple of 2^(e-7)), so every sum and difference -- exact, or
// rounded to binary32, whose ulp is then at least 2^-109 -- is a multiple of
// 2^-110 and never subnormal: the flushes are no-ops and DAZ has nothing to
// clear.  A wave holding a smaller nonzero input takes the flushing path.
//
// BC > 0 fixes the block at compile time: every stage then runs
// unconditionally and the compiler renames registers from stage to stage,
// where a run-time block keeps the values in place across the optional
// stages at the cost of a register move per butterfly.
template <bool kFlush, int BC = 0>
__device__ __forceinline__ void butterflies(float* v, int b) {
  if (BC) b = BC;
#pragma unroll
  for (int h = 1; h < kHalf; h *= 2) {
    if (h < b) {
#pragma unroll
      for (int j = 0; j < kHalf; ++j) {
        if (j & h) continue;
        const float a = v[j], c = v[j + h];
        v[j] = kFlush ? fadd(a, c) : a + c;
        v[j + h] = kFlush ? fsub(a, c) : a - c;
      }
    }
  }
  if (b > kHalf) {
    // stage 64 pairs token t (lower lane, v[t]) with token t + 64 (upper
    // lane, v[t]).  v_permlane32_swap(x, y) exchanges lanes 32..63 of x
    // with lanes 0..31 of y; applied to registers j and j + 32 it leaves
    // in every lane the two operands of one butterfly: lower lanes get
    // tokens (j, j + 64), upper lanes tokens (j + 32, j + 96), as (x, y).
    // The sum and difference stay where they are, so afterwards register
    // i of half h holds token tok_after(b, h, i).
#pragma unroll
    for (int j = 0; j < kHalf / 2; ++j) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[j]),
                                                        __float_as_uint(v[j + kHalf / 2]), false,
                                                        false);
      const float a = __uint_as_float(sw[0]), c = __uint_as_float(sw[1]);
      v[j] = kFlush ? fadd(a, c) : a + c;
      v[j + kHalf / 2] = kFlush ? fsub(a, c) : a - c;
    }
  }
}

// Token (0..127 in the tile) held in register i of lane half h after the
// butterflies: 64 h + i below block 128; after stage 64 the lower half
// holds tokens 0..31 and 64..95, the upper half 32..63 and 96..127.
__device__ __forceinline__ int tok_after(int b, int h, int i) {
  return b > kHalf ? i + 32 * h + (i >= kHalf / 2 ? kHalf / 2 : 0) : kHalf * h + i;
}

// tile_ok: the row phase found every nonzero value of the tile >= 2^-103
// (uniform over the work-group).  tail(v) runs the rest of the kernel on
// the rotated values inside each of the three forms, so their results
// never meet in one set of registers (a join would cost a register copy
// per value).
template <class Tail>
__device__ __forceinline__ void column_wht(const uint8_t* lds, int col, int half, int b,
                                           bool tile_ok, Tail&& tail) {
  float v[kHalf];
#pragma unroll
  for (int r = 0; r < kHalf; ++r) {
    const uint32_t h =
        *reinterpret_cast<const uint16_t*>(lds + (kHalf * half + r) * kRowBytes + 2 * col);
    v[r] = __uint_as_float(h << 16);
  }
  if (!tile_ok) {
#pragma unroll
    for (int r = 0; r < kHalf; ++r) v[r] = flush(v[r]);
    butterflies<true>(v, b);
    tail(v);
  } else if (b == kRows) {
    butterflies<false, kRows>(v, b);
    tail(v);
  } else {
    butterflies<false>(v, b);
    tail(v);
  }
}

__global__ __launch_bounds__(256) void k_dy_stats(const uint16_t* __restrict__ dy,
                                                  const float* __restrict__ sw, int64_t M,
                                                  int64_t N, int b, float* __restrict__ part_g,
                                                  float* __restrict__ part_v,
                                                  float* __restrict__ bmax) {
  constexpr int kTileBytes = kRows * kRowBytes;
  constexpr int kTrBytes = kHalf * kTrStride * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTileBytes > kTrBytes ? kTileBytes : kTrBytes];
  __shared__ float wmax[4];
  __shared__ int wok[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * kRows, c0 = (int64_t)blockIdx.x * kCols;
  // this tile's run of 128 rows x 2 nodes in the tile-by-tile node arrays
  const int64_t tbase = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256;

  // row phase: g leaves and their node(6) per 64 columns
  const int cg = t & 15, rb = t >> 4;
  const int64_t colv = c0 + 8 * cg;
  float s8[8];
  load_steps(sw, N, colv, s8);
  u32x4 raw[kRows / 16];
  load_rows(dy, N, m0, colv, rb, raw);
  u16x2 lo = {0xffff, 0xffff};
#pragma unroll
  for (int i = 0; i < kRows / 16; ++i) lo = tiny_min(lo, raw[i]);
  const bool wave_tiny_ok = __all(tiny_ok(lo));
  const bool fast = wave_tiny_ok && __all(steps_ok(s8));
  float mx = 0.0f;
#pragma unroll
  for (int i = 0; i < kRows / 16; ++i) {
    const int r = rb + 16 * i;
    st16(lds + r * kRowBytes + 16 * cg, raw[i]);
    float f[8];
    if (fast) {
      // |fl(x s)| = fl(|x| |s|): the sign bits are dropped before the product
      const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = __uint_as_float((w[k] & 0x7fffu) << 16) * fabs_bits(s8[2 * k]);
        f[2 * k + 1] = __uint_as_float(w[k] & 0x7fff0000u) * fabs_bits(s8[2 * k + 1]);
      }
    } else {
      unpack_bf16x8(raw[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = fabs_bits(fmul(f[e], s8[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, f[e]);
    const float node = wave_tree_partial<false>(reg_tree<false, 8>(f), 8);
    if ((cg & 7) == 0 && colv < N) part_g[tbase + 2 * r + (cg >> 3)] = node;
  }
  mx = wave_max(mx);
  if (lane == 0) {
    wmax[wave] = mx;
    wok[wave] = wave_tiny_ok ? 1 : 0;
  }
  __syncthreads();
  if (t == 0)
    bmax[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] =
        fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool tile_ok = wok[0] && wok[1] && wok[2] && wok[3];

  // column phase
  const int ccol = 32 * wave + (lane & 31), half = lane >> 5;
  column_wht(lds, ccol, half, b, tile_ok, [&](const float* v) {
  __syncthreads();  // every column read: the tile memory is reused below
  // v to row order, 64 rows at a time: the half-p lanes write their 64
  // tokens, then lane t reads row t >> 2, columns 32 (t & 3) .. +31, takes
  // |v| as the abs modifiers of the tree's first adds, and the lane pairs
  // (t, t ^ 1) join their 32-column nodes into node(6)
  float* tr = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // tokens 64 p .. 64 p + 63 to rows 0..63 of the transpose
    if (b > kHalf) {
#pragma unroll
      for (int j = 0; j < kHalf / 2; ++j)
        tr[(tok_after(b, half, (kHalf / 2) * p + j) - kHalf * p) * kTrStride + ccol] =
            v[(kHalf / 2) * p + j];
    } else if (half == p) {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) tr[i * kTrStride + ccol] = v[i];
    }
    __syncthreads();
    const int r = t >> 2, c32 = (t & 3) * 32;
    float a[16];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 x4 = *reinterpret_cast<const float4*>(&tr[r * kTrStride + c32 + 4 * q]);
      a[2 * q] = fabsf(x4.x) + fabsf(x4.y);
      a[2 * q + 1] = fabsf(x4.z) + fabsf(x4.w);
    }
    float node = reg_tree<false, 16>(a);
    node = node + dpp_xor1(node);  // non-negative leaves: no flush needed
    const int64_t cc = c0 + c32;
    if ((t & 1) == 0 && cc < N) part_v[tbase + 2 * (kHalf * p + r) + (c32 >> 6)] = node;
    __syncthreads();
  }
  });
}

__global__ __launch_bounds__(256) void k_dy_codes(const uint16_t* __restrict__ dy,
                                                  const float* __restrict__ sw, int64_t M,
                                                  int64_t N, int b,
                                                  const float* __restrict__ sr4,
                                                  int8_t* __restrict__ q_g,
                                                  int8_t* __restrict__ q_vt) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kRows * kRowBytes];
  __shared__ int wok[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * kRows, c0 = (int64_t)blockIdx.x * kCols;
  const float r_g = sr4[1], r_v = sr4[3];

  const int cg = t & 15, rb = t >> 4;
  const int64_t colv = c0 + 8 * cg;
  float s8[8];
  load_steps(sw, N, colv, s8);
  u32x4 raw[kRows / 16];
  load_rows(dy, N, m0, colv, rb, raw);
  u16x2 lo = {0xffff, 0xffff};
#pragma unroll
  for (int i = 0; i < kRows / 16; ++i) lo = tiny_min(lo, raw[i]);
  const bool wave_tiny_ok = __all(tiny_ok(lo));
  const bool fast = wave_tiny_ok && __all(steps_ok(s8));
  int8_t* qg_row = q_g + (m0 + rb) * N + colv;  // steps by 16 N per row
  const int64_t qg_step = 16 * N;
#pragma unroll
  for (int i = 0; i < kRows / 16; ++i, qg_row += qg_step) {
    const int r = rb + 16 * i;
    st16(lds + r * kRowBytes + 16 * cg, raw[i]);
    if (colv < N) {
      float f[8];
      if (fast) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[2 * k] = __uint_as_float(w[k] << 16) * s8[2 * k];
          f[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u) * s8[2 * k + 1];
        }
      } else {
        unpack_bf16x8(raw[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = fmul(f[e], s8[e]);
      }
      uint32_t p[2] = {0, 0};
#pragma unroll
      for (int e = 0; e < 8; e += 4) p[e >> 2] = quant_pack4(f[e], f[e + 1], f[e + 2], f[e + 3], r_g);
      *reinterpret_cast<uint2*>(qg_row) = make_uint2(p[0], p[1]);
    }
  }
  if (lane == 0) wok[wave] = wave_tiny_ok ? 1 : 0;
  __syncthreads();
  const bool tile_ok = wok[0] && wok[1] && wok[2] && wok[3];
  const int ccol = 32 * wave + (lane & 31), half = lane >> 5;
  column_wht(lds, ccol, half, b, tile_ok, [&](const float* v) {
  // The codes go through LDS as [column][token] (after the barrier no lane
  // reads the bf16 tile any more), so that each store instruction writes
  // whole 128-token runs of 8 columns instead of 16-byte pieces of 64.
  // Columns past N are computed from the zero tile and not stored.
  constexpr int kCodeStride = kRows + 16;  // padded bytes per column
  static_assert(kCols * kCodeStride <= kRows * kRowBytes, "codes fit the tile memory");
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kHalf / 16; ++p) {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      w[i >> 2] = quant_pack4(v[16 * p + i], v[16 * p + i + 1], v[16 * p + i + 2], v[16 * p + i + 3], r_v);
    // registers 16 p .. 16 p + 15 hold 16 consecutive tokens
    st16(lds + ccol * kCodeStride + tok_after(b, half, 16 * p), u32x4{w[0], w[1], w[2], w[3]});
  }
  __syncthreads();
  // lane t stores 16 tokens of columns (t >> 3) + 32 k: 32 M apart in q_vt
  int8_t* vt = q_vt + (c0 + (t >> 3)) * M + m0 + 16 * (t & 7);
  const int64_t vt_step = 32 * M;
#pragma unroll
  for (int k = 0; k < kCols * kRows / 16 / 256; ++k, vt += vt_step) {
    const int c = k * 32 + (t >> 3), ch = 16 * (t & 7);
    if (c0 + c < N) st16(vt, *reinterpret_cast<const u32x4*>(lds + c * kCodeStride + ch));
  }
  });
}

}  // namespace

bool dy_fused_ok(int dtype, int64_t M, int64_t N, int block) {
  return dtype == BRQ_BF16 && M % kRows == 0 && N % 64 == 0 && block >= 1 && block <= kRows &&
         M > 0 && N > 0;
}

size_t dy_fused_ws(int64_t M, int64_t N, int chunk_log2) {
  const int64_t P = M * (N / 64);
  const int64_t PT = tile_map_size(M, N / 64);  // tile-by-tile node arrays
  const int64_t nblk = cdiv(N, kCols) * (M / kRows);
  return 2 * align256((size_t)(PT > 0 ? PT : 1) * sizeof(float)) +
         align256((size_t)(nblk > 0 ? nblk : 1) * sizeof(float)) +
         flat_reduce_pair_ws(P, chunk_log2) + 256;
}

hipError_t quantize_dy_fused(const void* dy, int64_t M, int64_t N, const float* sw, int block,
                             int8_t* q_g, float* s_g, float* amax_g, int8_t* q_vt, float* s_v,
                             void* ws, int chunk_log2, int32_t* dflags, hipStream_t s) {
  const int64_t nb = N / 64;
  const int64_t P = M * nb;
  const int64_t PT = tile_map_size(M, nb);
  const int64_t gx = cdiv(N, kCols), gy = M / kRows;
  char* w = (char*)ws;
  float* part_g = (float*)w;
  w += align256((size_t)PT * sizeof(float));
  float* part_v = (float*)w;
  w += align256((size_t)PT * sizeof(float));
  float* bmax = (float*)w;
  w += align256((size_t)(gx * gy) * sizeof(float));
  void* fws = w;
  w += flat_reduce_pair_ws(P, chunk_log2);
  float* sc = (float*)w;  // [0,1] g sum/max, [2,3] v sum/max, [4..7] s_g r_g s_v r_v
  dim3 g((unsigned)gx, (unsigned)gy), b(256);
  hipLaunchKernelGGL(k_dy_stats, g, b, 0, s, (const uint16_t*)dy, sw, M, N, block, part_g, part_v,
                     bmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // both step sizes and the max of |g| come from the reduction's two
  // final work-groups
  const float inv_n = 1.0f / (float)(M * N);  // host binary32 division, correctly rounded
  const PairFin fin{1, inv_n, sc + 4, s_g, s_v, amax_g, bmax, gx * gy};
  int lognb = -1;
  if ((nb & (nb - 1)) == 0)
    for (lognb = 0; (int64_t(1) << lognb) < nb;) ++lognb;
  const TileMap tm{nb, gx, lognb};
  if ((e = flat_reduce_pair(part_g, part_v, P, sc, sc + 2, fws, chunk_log2, dflags, s, &fin,
                            &tm)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(k_dy_codes, g, b, 0, s, (const uint16_t*)dy, sw, M, N, block, sc + 4, q_g,
                     q_vt);
  return hipGetLastError();
}

}  // namespace brq
