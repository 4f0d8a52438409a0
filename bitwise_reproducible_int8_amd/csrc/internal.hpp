// internal.hpp -- launcher declarations shared by the libbrq translation
// units (host side).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/brq.h"

namespace brq {

// Sizes of scratch regions, in bytes, rounded up to 256.
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Leaves per work-group of the flat tree reductions.
int flat_chunk_log2(const brq_tune* t);

// ---- canonical-tree reductions over a flat array -------------------------
// Leaf kinds of the first pass.
enum LeafKind { LEAF_ABS = 0, LEAF_ABS_COLMUL = 1, LEAF_SQUARE = 2, LEAF_RAW = 3 };

// Workspace needed to reduce n leaves to one value (partials of every level
// plus the small scalar block).
size_t flat_reduce_ws(int64_t n, int chunk_log2);

// Reduce n leaves of kind `leaf` (dtype of x) to the tree sum; writes the
// sum and the max of |leaf| into out[0], out[1] (device), raising
// BRQ_FLAG_NONFINITE when the sum is not finite.  Uses ws.
// wht_block > 0 (leaf LEAF_ABS_COLMUL): the leaves are |x * col_mul| after
// the Walsh-Hadamard rotation along each row in blocks of wht_block
// (cols % wht_block == 0, wht_block <= 128); the chunk is then fixed.
// fin (optional): the scalar step the caller would launch after the sum,
// run by the final work-group instead (same operations, same order).
enum FinKind { FIN_NONE = 0, FIN_LSQ = 1, FIN_NORM = 2 };
struct FlatFin {
  int kind;
  float inv_n;   // FIN_LSQ: s = fl(fl(S * inv_n) * K2), r = fl(1/s) (0 when s == 0)
  float* sr;     // FIN_LSQ: {s, r}
  float* scale;  // FIN_LSQ: s (optional)
  float* amax;   // FIN_LSQ: the max (optional)
  float* sumsq;  // FIN_NORM: S
  float* norm;   // FIN_NORM: fl(sqrt S)
};
hipError_t flat_reduce(const void* x, int dtype, int leaf, const float* col_mul,
                       int64_t n, int64_t cols, float* out2, void* ws,
                       int chunk_log2, int32_t* dflags, hipStream_t s, int wht_block = 0,
                       const FlatFin* fin = nullptr);

// Two raw fp32 leaf arrays of equal length n reduced as two flat_reduce
// calls would, in one launch per level; workspace flat_reduce_pair_ws.
size_t flat_reduce_pair_ws(int64_t n, int chunk_log2);
// Storage of a leaf array kept tile by tile: leaf i = (row, c) of a
// row-major [rows][nb] array (row = i / nb, c = i % nb) sits at
// ((row / 128) gx + c / 2) 256 + (row % 128) 2 + c % 2, i.e. each 128-row x
// 2-column tile is one contiguous run of 256 values.  The tree is still the
// one over the row-major order.  lognb = log2(nb) when nb is a power of
// two, else -1.
struct TileMap {
  int64_t nb;
  int64_t gx;
  int lognb;
};
inline int64_t tile_map_size(int64_t rows, int64_t nb) {
  return ((rows + 127) / 128) * ((nb + 1) / 2) * 256;
}
// fin (optional): both LSQ steps from the two sums -- sr4 = {s0, r0, s1, r1},
// s0/s1 copies -- and amax0 = the max over bmax[0 .. nb) (order-free), run
// by the two final work-groups.
struct PairFin {
  int on;
  float inv_n;
  float* sr4;
  float* s0;
  float* s1;
  float* amax0;
  const float* bmax;
  int64_t nb;
};
// tm (optional): both leaf arrays are stored tile by tile (TileMap).
hipError_t flat_reduce_pair(const float* x0, const float* x1, int64_t n, float* out0,
                            float* out1, void* ws, int chunk_log2, int32_t* dflags,
                            hipStream_t s, const PairFin* fin = nullptr,
                            const TileMap* tm = nullptr);

// Optimizer step (optim.hip).
hipError_t adamw_decide(const float* norm, float max_norm, float spike, int skip_steps,
                        int32_t* skip_state, float* ctl, int32_t* dflags, hipStream_t s);
hipError_t adamw_step(void* param, int pdtype, const void* grad, int gdtype, float* m, float* v,
                      int64_t n, const brq_adamw_hparams& h, const float* ctl, hipStream_t s);

// From a tree sum on device, compute the LSQ step size and reciprocal:
// sr[0] = s, sr[1] = r.  Optionally copies s and the max into scale/amax.
hipError_t lsq_finalize(const float* sum_max, float inv_n, float* sr,
                        float* scale, float* amax, hipStream_t s);

// Elementwise quantisation with the device reciprocal sr[1].
hipError_t quant_flat(const void* x, int dtype, const float* col_mul, int64_t n,
                      int64_t cols, const float* sr, int8_t* q, hipStream_t s);

// Per-row quantisation (one wave per row).
hipError_t quant_rows(const void* x, int dtype, int64_t rows, int64_t cols,
                      int8_t* q, float* scale, float* amax, int32_t* dflags,
                      hipStream_t s);
// Per-row quantisation (and transposes) of count tensors in a few grouped
// launches; jobs validated by the caller, count <= BRQ_ROWS_MULTI_MAX.
hipError_t quant_rows_multi(const brq_rows_job* jobs, int count, int32_t* dflags, hipStream_t s);

// Exact-sum statistic (exact.hip): per-tensor S and max |v| into out2[0..1]
// (two launches), and the per-row quantiser with exact row statistics.
// Attention forward with an int8 P.V product (attn.hip).
hipError_t attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t Hq,
                    int64_t Hkv, int64_t T, int64_t d, int64_t window, float* o, int32_t* dflags,
                    hipStream_t s);

// Rows rotation of dY * s_w and its codes (dxwht.hip).
size_t wht_rows_ws(int64_t M, int64_t N);
hipError_t wht_rows_quant(const void* dy, int dtype, int64_t M, int64_t N, const float* s_w,
                          int block, int8_t* q_g, float* s_g, float* sr, void* ws,
                          int32_t* dflags, hipStream_t s);

size_t exact_reduce_ws(int64_t n);
hipError_t exact_reduce(const void* x, int dtype, const float* col_mul, int64_t n, int64_t cols,
                        float* out2, void* ws, int32_t* dflags, hipStream_t s);
hipError_t quant_rows_exact(const void* x, int dtype, int64_t rows, int64_t cols, int8_t* q,
                            float* scale, float* amax, int32_t* dflags, hipStream_t s);

// int8 transpose: q [rows][cols] -> qt [cols][rows].
hipError_t transpose_i8(const int8_t* q, int64_t rows, int64_t cols, int8_t* qt,
                        hipStream_t s);

// ---- GEMMs ------------------------------------------------------------------
enum EpiKind { EPI_FWD = 0, EPI_SCALAR = 1, EPI_DW = 2 };
struct EpiArgs {
  int kind;
  const float* s0;   // fwd: s_x   scalar: s     dw: s_x
  const float* s1;   // fwd: s_w   dw: s_u
  const float* s2;   // dw: s_v
  int per_row;       // fwd: s_w is per output column
  float inv_b;       // dw: exact 2^-log2(block)
  int out_bf16 = 0;  // C holds bf16 (round to nearest even) instead of fp32
};
size_t gemm_ws(int64_t I, int64_t J, int64_t Kc, const brq_tune* t);
// C[i][j] = epi(sum_k A[i][k] * B[j][k]); A [I][Kc], B [J][Kc], C [I][J].
hipError_t gemm_i8(const int8_t* A, const int8_t* B, int64_t I, int64_t J,
                   int64_t Kc, float* C, const EpiArgs& epi, void* ws,
                   size_t ws_bytes, const brq_tune* t, hipStream_t s);

// ---- Walsh-Hadamard rotations ----------------------------------------------
size_t wht_x_ws(int64_t M, int64_t K, int block);
// Per-tensor LSQ codes of x and the integer rotation of those codes in one
// call (one read of x for the codes and the rotation's statistic).
size_t quant_x_wht_ws(int64_t M, int64_t K, int block, int chunk_log2);
hipError_t quantize_x_wht(const void* x, int dtype, int64_t M, int64_t K, int block,
                          int8_t* q_x, float* s_x, float* amax_x, int8_t* q_ut, float* s_u,
                          void* ws, int chunk_log2, int32_t* dflags, hipStream_t s);
size_t wht_dy_ws(int64_t M, int64_t N, int block, int chunk_log2);
hipError_t wht_quant_x(const int8_t* q_x, int64_t M, int64_t K, int block,
                       int8_t* q_ut, float* s_u, void* ws, hipStream_t s);
hipError_t wht_quant_dy(const void* dy, int dtype, int64_t M, int64_t N,
                        int block, int8_t* q_vt, float* s_v, void* ws,
                        int chunk_log2, int32_t* dflags, hipStream_t s);

// ---- both backward codes of dY in two passes (dy.hip) -------------------------
bool dy_fused_ok(int dtype, int64_t M, int64_t N, int block);
size_t dy_fused_ws(int64_t M, int64_t N, int chunk_log2);
hipError_t quantize_dy_fused(const void* dy, int64_t M, int64_t N, const float* sw, int block,
                             int8_t* q_g, float* s_g, float* amax_g, int8_t* q_vt, float* s_v,
                             void* ws, int chunk_log2, int32_t* dflags, hipStream_t s);

// ---- RMSNorm / grad-norm ------------------------------------------------------
hipError_t rmsnorm_fwd(const void* x, const void* g, int dtype, int64_t T,
                       int64_t D, float eps, void* y, float* rstd,
                       int32_t* dflags, hipStream_t s);
int rmsnorm_bwd_rows(int64_t D, int dtype, const brq_tune* t);
size_t rmsnorm_bwd_ws(int64_t T, int64_t D, int dtype, const brq_tune* t);
hipError_t rmsnorm_bwd(const void* x, const void* g, const float* rstd,
                       const void* dy, int dtype, int64_t T, int64_t D,
                       void* dx, float* dg, void* ws, const brq_tune* t,
                       hipStream_t s);
hipError_t grad_norm(const float* v, int64_t n, float* sumsq, float* norm,
                     void* ws, int chunk_log2, int32_t* dflags, hipStream_t s);

// ---- deterministic gradient exchange (exchange.hip) ------------------------------
// parts: host array of R*S*A device pointers in mesh order.
hipError_t dp_reduce(const float* const* parts, int R, int S, int A, int64_t n, int average,
                     float* out, int32_t* dflags, hipStream_t s);

// ---- binary32 primitives over a range of bit patterns (primitive.hip) -------------
hipError_t fp32_primitive(int prim, uint32_t first, int64_t count, uint32_t* out, hipStream_t s);

// ---- hash ------------------------------------------------------------------------
size_t hash_ws(const brq_tensor_ref* t, int n);
size_t hash_digests_ws(const brq_tensor_ref* t, int n);
hipError_t hash_tensor_digests(const brq_tensor_ref* t, int n, uint8_t* digests, void* ws,
                               hipStream_t s);
hipError_t hash_combine(const uint8_t* digests, int n, uint8_t* digest32, hipStream_t s);
hipError_t hash_tensor_leaves(const brq_tensor_ref* t, int n, void* ws, hipStream_t s);
hipError_t hash_tensor_finish(const brq_tensor_ref* t, int n, uint8_t* digests, void* ws,
                              hipStream_t s);
hipError_t hash_state(const brq_tensor_ref* t, int n, uint8_t* digest32,
                      void* ws, hipStream_t s);

}  // namespace brq
