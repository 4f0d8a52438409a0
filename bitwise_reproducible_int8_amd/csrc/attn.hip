// attn.hip -- attention forward with an int8 P.V product (a variant; Open-1B
// report §3.2 "int8 computation": inside flash attention the P.V product
// quantises the attention weights and values to int8 per block and
// multiplies them as integers, while the QK^T logits and the softmax stay in
// higher precision; §3.1: grouped-query attention, causal, sliding window).
//
// Definitions (every floating-point step one rounded, flushed binary32
// operation, in this order):
//   S_ij = fl(dot_ij * c), c = fl(1/fl(sqrt d)); dot_ij sequential over e of
//          the exact bf16 products
//   key j visible from query i iff i - window < j <= i
//   64-key blocks in ascending order; per row m = max(m, block max),
//   a = exp_f(m_old - m) (0 while m_old = -inf), p = exp_f(S - m) (0 hidden),
//   l = fl(fl(l * a) + pairwise tree of the block's 64 p)
//   P tile 64 x 64: s_p = fl(max p * fl(1/127)); V block 64 x d:
//   s_v = fl(max |v| * fl(1/127)); codes clamp(rint(fl(x * fl(1/s))), +-127)
//   o = fl(fl(o * a) + fl(fl(sum_j qp qv) * fl(s_p * s_v))) (exact integer
//   sum), finally o = fl(o * fl(1/l)); a row with no visible key in a block
//   is left as it was.
//
// One work-group (256 lanes) per (query head, 64-query block).  Q^T and
// K^T sit in LDS as fp32 [d][64]; each lane owns a 4 x 4 block of logits
// (rows 4 (t >> 4) .., keys 4 (t & 15) ..) and runs the sequential dot over
// e with fused multiply-adds: a bf16 product is exact, so fma(q, k, acc) is
// fl(acc + q k); when every nonzero q, k is >= 2^-50 in magnitude, every
// product and partial sum is a multiple of 2^-114 and never subnormal (the
// flushes are identities), else the block takes the flushing form.  The 16
// lanes of a row group share the row's maximum, exp and tree by xor
// butterflies within the group.  P codes [64][64] and V codes [d][64] go to
// LDS; each lane owns one row and 32 consecutive e of the output, whose
// integer products are v_dot4 sums (exact, like the matrix cores').
#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

constexpr int kBlk = 64;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// exp for x <= 0: Cody-Waite reduction by ln 2 (15-bit head, exact n*head),
// degree-7 Taylor polynomial in Horner form, exact scaling by 2^n.
__device__ __forceinline__ float exp_f(float x) {
  if (!(x >= -104.0f)) return 0.0f;
  const float inv_ln2 = __uint_as_float(0x3fb8aa3bu);
  const float ln2_hi = __uint_as_float(0x3f317200u);
  const float ln2_lo = __uint_as_float(0x35bfbe8eu);
  const float n = __builtin_rintf(fmul(x, inv_ln2));
  const float r = fsub(fsub(x, fmul(n, ln2_hi)), fmul(n, ln2_lo));
  float p = 1.0f / 5040.0f;
  p = fadd(fmul(p, r), 1.0f / 720.0f);
  p = fadd(fmul(p, r), 1.0f / 120.0f);
  p = fadd(fmul(p, r), 1.0f / 24.0f);
  p = fadd(fmul(p, r), 1.0f / 6.0f);
  p = fadd(fmul(p, r), 0.5f);
  p = fadd(fmul(p, r), 1.0f);
  p = fadd(fmul(p, r), 1.0f);
  const int ni = (int)n;
  if (ni < -126) return 0.0f;
  return fmul(p, __uint_as_float((uint32_t)(ni + 127) << 23));
}

// The same value without the flushes when they cannot act: for x = 0 or
// |x| >= 2^-100 the reduced argument r is 0 or at least 2^-100 in
// magnitude (|x - n ln 2| for a binary32 x in [-104, 0] is never that
// small otherwise), so every Horner product and sum is 0 or normal; only
// the final scaling can land below 2^-126 and keeps its flush.
__device__ __forceinline__ float exp_f_fast(float x) {
  if (x != 0.0f && fabsf(x) < 0x1p-100f) return exp_f(x);
  if (!(x >= -104.0f)) return 0.0f;
  const float inv_ln2 = __uint_as_float(0x3fb8aa3bu);
  const float ln2_hi = __uint_as_float(0x3f317200u);
  const float ln2_lo = __uint_as_float(0x35bfbe8eu);
  const float n = __builtin_rintf(x * inv_ln2);
  const float r = (x - n * ln2_hi) - n * ln2_lo;
  float p = 1.0f / 5040.0f;
  p = p * r + 1.0f / 720.0f;
  p = p * r + 1.0f / 120.0f;
  p = p * r + 1.0f / 24.0f;
  p = p * r + 1.0f / 6.0f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  const int ni = (int)n;
  if (ni < -126) return 0.0f;
  return fmul(p, __uint_as_float((uint32_t)(ni + 127) << 23));
}

__device__ __forceinline__ int8_t code_of(float x, float r) { return (int8_t)quant_code(x, r); }

// max over the 16 lanes of a row group (xor 1, 2, 4, 8: inside the group)
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void k_attn_fwd(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v, int64_t T,
                                                  int group, int64_t window, float c,
                                                  float* __restrict__ o, int32_t* flags) {
  __shared__ float qT[D][kBlk];
  __shared__ float kT[D][kBlk];
  __shared__ __attribute__((aligned(16))) int8_t pc[kBlk][kBlk];
  __shared__ __attribute__((aligned(16))) int8_t vT[D][kBlk];
  __shared__ float s_alpha[kBlk], s_l[kBlk];
  __shared__ int s_any[kBlk];
  __shared__ float red[8];
  __shared__ int s_slow[2];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // the last query blocks see the most key blocks: they start first
  const int64_t qb = (int64_t)gridDim.x - 1 - blockIdx.x, h = blockIdx.y, hk = h / group;
  const uint16_t* Q = q + (h * T + qb * kBlk) * D;
  const uint16_t* K = k + hk * T * D;
  const uint16_t* V = v + hk * T * D;
  constexpr int kChunks = kBlk * D / 8;  // 16-byte chunks of a 64-row tile

  // Q^T into LDS (chunk c: row c % 64, columns 8 (c / 64) ..), and the
  // fast-path test of its values
  bool small = false;  // some nonzero |q| < 2^-50 in this lane
  for (int cidx = t; cidx < kChunks; cidx += 256) {
    const int row = cidx & 63, e0 = (cidx >> 6) * 8;
    float f[8];
    unpack_bf16x8(ld16(Q + row * D + e0), f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      qT[e0 + u][row] = f[u];
      small = small || (f[u] != 0.0f && fabsf(f[u]) < 0x1p-50f);
    }
  }
  if (t < 2) s_slow[t] = 0;
  __syncthreads();
  if (small) s_slow[0] = 1;

  // per-row state: the lanes of row group rg hold rows 4 rg .. 4 rg + 3
  const int rg = t >> 4, kg = t & 15;
  float m[4], l[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) { m[a] = -INFINITY; l[a] = 0.0f; }
  // output lane map: row t >> 2, columns (t & 3) * (D / 4) ..
  constexpr int kOut = D / 4;
  const int orow = t >> 2, ocol = (t & 3) * kOut;
  float acc[kOut];
#pragma unroll
  for (int e = 0; e < kOut; ++e) acc[e] = 0.0f;

  const int64_t i_lo = qb * kBlk;
  for (int64_t kb = 0; kb <= qb; ++kb) {
    if (kb * kBlk + kBlk - 1 <= i_lo - window) continue;  // no query sees this block
    const uint16_t* Kb = K + kb * kBlk * D;
    const uint16_t* Vb = V + kb * kBlk * D;
    // K^T into LDS, V block's absmax
    bool ksmall = false;
    float vmax = 0.0f;
    for (int cidx = t; cidx < kChunks; cidx += 256) {
      const int row = cidx & 63, e0 = (cidx >> 6) * 8;
      float f[8], g[8];
      unpack_bf16x8(ld16(Kb + row * D + e0), f);
      unpack_bf16x8(ld16(Vb + row * D + e0), g);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        kT[e0 + u][row] = f[u];
        ksmall = ksmall || (f[u] != 0.0f && fabsf(f[u]) < 0x1p-50f);
        vmax = fmaxf(vmax, fabs_bits(g[u]));
      }
    }
    vmax = wave_max(vmax);
    if (lane == 0) red[wave] = vmax;
    if (ksmall) s_slow[1] = 1;
    __syncthreads();
    const bool slow = s_slow[0] || s_slow[1];
    vmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    // logits of the lane's 4 x 4 block
    float s[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) s[a][b] = 0.0f;
    if (!slow) {
#pragma unroll 4
      for (int e = 0; e < D; ++e) {
        const float4 qa = *reinterpret_cast<const float4*>(&qT[e][4 * rg]);
        const float4 kv = *reinterpret_cast<const float4*>(&kT[e][4 * kg]);
        const float qv4[4] = {qa.x, qa.y, qa.z, qa.w}, kv4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) s[a][b] = __builtin_fmaf(qv4[a], kv4[b], s[a][b]);
      }
    } else {
      for (int e = 0; e < D; ++e) {
        const float4 qa = *reinterpret_cast<const float4*>(&qT[e][4 * rg]);
        const float4 kv = *reinterpret_cast<const float4*>(&kT[e][4 * kg]);
        const float qv4[4] = {qa.x, qa.y, qa.z, qa.w}, kv4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) s[a][b] = fadd(s[a][b], fmul(qv4[a], kv4[b]));
      }
    }
    // scale and mask; block maximum per row
    float bmax[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t gi = i_lo + 4 * rg + a;
      bmax[a] = -INFINITY;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t gj = kb * kBlk + 4 * kg + b;
        // without the slow inputs every nonzero logit is a multiple of
        // 2^-114, so s * c (c = 1/sqrt(d) > 2^-4) is 0 or above 2^-118 and
        // its flush cannot act
        const float sc = slow ? fmul(s[a][b], c) : s[a][b] * c;
        s[a][b] = (gj > gi || gj <= gi - window) ? -INFINITY : sc;
        bmax[a] = fmaxf(bmax[a], s[a][b]);
      }
      bmax[a] = group16_max(bmax[a]);
    }
    // rescale factors, probabilities, row sums (pairwise tree: in-lane
    // pairs, then the group's xor butterflies, which pair node(k, 2i) with
    // node(k, 2i+1) at every level)
    float pmax = 0.0f;
    float pr[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const bool any = bmax[a] != -INFINITY;
      const float mn = fmaxf(bmax[a], m[a]);
      const float alpha = !any ? 1.0f : (m[a] == -INFINITY ? 0.0f : exp_f_fast(fsub(m[a], mn)));
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        pr[a][b] = (!any || s[a][b] == -INFINITY) ? 0.0f : exp_f_fast(fsub(s[a][b], mn));
        pmax = fmaxf(pmax, pr[a][b]);
      }
      // the probabilities are +0 or normal and non-negative, so no partial
      // sum of the tree can be subnormal: plain adds equal flushed ones
      float node = (pr[a][0] + pr[a][1]) + (pr[a][2] + pr[a][3]);
#pragma unroll
      for (int o2 = 1; o2 < 16; o2 <<= 1) node = node + __shfl_xor(node, o2);
      if (any) {
        l[a] = fadd(fmul(l[a], alpha), node);
        m[a] = mn;
      }
      if (kg == 0) {
        s_alpha[4 * rg + a] = alpha;
        s_any[4 * rg + a] = any ? 1 : 0;
      }
    }
    pmax = wave_max(pmax);
    __syncthreads();  // every lane is done with red (vmax) and kT
    if (lane == 0) red[4 + wave] = pmax;
    __syncthreads();
    pmax = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
    const float inv127 = 1.0f / 127.0f;
    const float sp = fmul(pmax, inv127), sv = fmul(vmax, inv127);
    const float rp = sp == 0.0f ? 0.0f : fl_div(1.0f, sp);
    const float rv = sv == 0.0f ? 0.0f : fl_div(1.0f, sv);
    // P codes
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= (uint32_t)(uint8_t)code_of(pr[a][b], rp) << (8 * b);
      *reinterpret_cast<uint32_t*>(&pc[4 * rg + a][4 * kg]) = w;
    }
    // V codes, transposed
    for (int cidx = t; cidx < kChunks; cidx += 256) {
      const int row = cidx & 63, e0 = (cidx >> 6) * 8;
      float g[8];
      unpack_bf16x8(ld16(Vb + row * D + e0), g);
#pragma unroll
      for (int u = 0; u < 8; ++u) vT[e0 + u][row] = code_of(g[u], rv);
    }
    __syncthreads();
    // integer products of the lane's row and columns, dequantised once
    const float cs = fmul(sp, sv);
    if (s_any[orow]) {
      const float alpha = s_alpha[orow];
      const int* prow = reinterpret_cast<const int*>(&pc[orow][0]);
#pragma unroll 4
      for (int e = 0; e < kOut; ++e) {
        const int* vcol = reinterpret_cast<const int*>(&vT[ocol + e][0]);
        int dot = 0;
#pragma unroll
        for (int j4 = 0; j4 < kBlk / 4; ++j4) dot = __builtin_amdgcn_sdot4(prow[j4], vcol[j4], dot, false);
        // fl(fl(dot) * cs) needs no flush: cs is flushed (0 or normal) and
        // a nonzero integer sum converts to a magnitude of at least 1
        acc[e] = fadd(fmul(acc[e], alpha), (float)dot * cs);
      }
    }
    __syncthreads();  // pc, vT, s_alpha, s_any reused by the next block
  }
  // final normalisation: the row sums go to LDS for the output lanes
  if (kg == 0) {
#pragma unroll
    for (int a = 0; a < 4; ++a) s_l[4 * rg + a] = l[a];
  }
  __syncthreads();
  const float lr = s_l[orow];
  const float il = fl_div(1.0f, lr);
  float* O = o + (h * T + qb * kBlk + orow) * D + ocol;
#pragma unroll
  for (int e = 0; e < kOut; e += 4) {
    f32x4 w4 = {fmul(acc[e], il), fmul(acc[e + 1], il), fmul(acc[e + 2], il),
                fmul(acc[e + 3], il)};
    *reinterpret_cast<f32x4*>(O + e) = w4;
  }
  if ((t & 3) == 0 && !__builtin_isfinite(lr)) set_flag(flags, BRQ_FLAG_NONFINITE);
}

}  // namespace

hipError_t attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t Hq,
                    int64_t Hkv, int64_t T, int64_t d, int64_t window, float* o, int32_t* dflags,
                    hipStream_t s) {
  const float c = 1.0f / sqrtf((float)d);  // host binary32: both steps correctly rounded
  dim3 g((unsigned)(T / kBlk), (unsigned)Hq), b(256);
  const int group = (int)(Hq / Hkv);
  if (d == 64)
    hipLaunchKernelGGL(k_attn_fwd<64>, g, b, 0, s, q, k, v, T, group, window, c, o, dflags);
  else
    hipLaunchKernelGGL(k_attn_fwd<128>, g, b, 0, s, q, k, v, T, group, window, c, o, dflags);
  return hipGetLastError();
}

}  // namespace brq
