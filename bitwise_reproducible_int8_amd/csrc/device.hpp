// device.hpp -- gfx950 device helpers for libbrq: the binary32 arithmetic
// model, bf16 conversion, and the canonical pairwise tree on 64-lane waves.
//
// Arithmetic model (Open-1B report, §2.1 "Fused multiply-add",
// "Subnormals" and Table 1): one IEEE binary32 operation per step, round to
// nearest even, never contracted (the library is built with
// -ffp-contract=off and this header repeats it as a pragma); fp32 denormals
// are kept by the hardware (IEEE mode) and every result that lands in the
// subnormal range is replaced by a zero of the same sign here, explicitly,
// as is every subnormal value read from memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace brq {

constexpr int kWave = 64;

// ---- binary32 model ------------------------------------------------------
__device__ __forceinline__ float flush(float v) {
  uint32_t u = __float_as_uint(v);
  return ((u & 0x7f800000u) == 0u) ? __uint_as_float(u & 0x80000000u) : v;
}
// A non-negative value: 0 or >= 2^-126 after the flush.
__device__ __forceinline__ float flush_nonneg(float v) {
  return (v < 1.17549435e-38f) ? 0.0f : v;
}
__device__ __forceinline__ float fadd(float a, float b) { return flush(a + b); }
__device__ __forceinline__ float fsub(float a, float b) { return flush(a - b); }
__device__ __forceinline__ float fmul(float a, float b) { return flush(a * b); }
// Division and square root: the correctly rounded binary32 operations (the
// library is built with -fhip-fp32-correctly-rounded-divide-sqrt), then the
// flush.  Every kernel divides and takes square roots through these two, and
// brq_fp32_primitive runs the same two on any range of inputs, so a sweep of
// all 2^32 binary32 patterns checks what the kernels execute.
__device__ __forceinline__ float fl_div(float a, float b) { return flush(a / b); }
__device__ __forceinline__ float fl_sqrt(float a) { return flush(__builtin_sqrtf(a)); }
__device__ __forceinline__ float fabs_bits(float a) {
  return __uint_as_float(__float_as_uint(a) & 0x7fffffffu);
}

// bf16 <-> fp32: widening is exact (then DAZ); narrowing rounds to nearest
// even on the bit pattern (a NaN stays a quiet NaN).
__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
  return flush(__uint_as_float(h16 << 16));
}
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two binary32 values rounded to bf16 (nearest even) by one conversion
// instruction (v_cvt_pk_bf16_f32), packed lo | hi << 16.  For every input
// that is not a NaN this is f32_to_bf16 of each (the instruction rounds to
// nearest even in the default mode and keeps subnormals); a NaN gives a
// quiet NaN whose payload may differ.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// LSQ factor 2 * fl(1/fl(sqrt(127))) as binary32 bits 0x3e35bb0a:
// fl(sqrt(127)) = 0x41344f93, its binary32 reciprocal 0x3db5bb0a, times 2.
__device__ __forceinline__ float lsq_k2() { return __uint_as_float(0x3e35bb0au); }

// q = clamp(rint(fl(v * r)), -127, 127), rounding half to even, returned
// as the low byte of a binary32 bit pattern.  The clamp comes first (one
// median of three): the bounds are integers and rint is monotone, so
// clamping before or after rounding gives the same integer.  Adding
// 1.5 * 2^23 to a value of magnitude at most 127 then lands in the binade
// [2^23, 2^24), whose spacing is 1: the add rounds to the nearest integer
// (ties to even) and the sum's bit pattern is 0x4b400000 + q, whose low
// byte is q as an int8.  The product is not flushed: a subnormal v * r and
// its flushed zero both give the code 0.  (A NaN product has no defined
// code.)
__device__ __forceinline__ uint32_t quant_code_bits(float v, float r) {
  const float t = __builtin_amdgcn_fmed3f(v * r, -127.0f, 127.0f);
  return __float_as_uint(t + 12582912.0f);
}
__device__ __forceinline__ int quant_code(float v, float r) {
  return (int)(int8_t)(quant_code_bits(v, r) & 0xffu);
}
// The codes of four values packed little-endian into one word (two byte
// permutes and an or).
__device__ __forceinline__ uint32_t quant_pack4(float v0, float v1, float v2, float v3, float r) {
  const uint32_t a = quant_code_bits(v0, r), b = quant_code_bits(v1, r);
  const uint32_t c = quant_code_bits(v2, r), d = quant_code_bits(v3, r);
  // v_perm_b32(S0, S1, sel): selector byte 0..3 takes byte of S1, 4..7 of
  // S0, 0x0c gives 0
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a0, b0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x04000c0cu);  // 0, 0, c0, d0
  return lo | hi;
}

// ---- wave-level canonical tree ---------------------------------------------
// Lane l holds node(j, l) of some level j for 64 consecutive nodes.  After
// the butterfly every lane holds node(j + 6, 0): at step s the partner lane
// is l ^ s, and because binary32 addition is commutative bit for bit the
// two partners compute the same value node(2i) + node(2i+1).
// The first four steps use DPP (quad permutes, half-row and row mirrors,
// valid because each group is uniform by then); the last two use one
// cross-lane swap each (lanes_16, lanes_32).
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_mirror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
}

// Both values of the lane pair (l, l ^ 16), resp. (l, l ^ 32), in every
// lane: v_permlane16_swap (v_permlane32_swap) of a register with itself
// swaps its odd 16-lane rows with the even ones (its upper 32 lanes with
// the lower), so the first result holds the value of the pair's lower lane
// and the second that of its upper lane.  One instruction, no LDS round
// trip.  Every lane of the wave must be active.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair lanes_16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair lanes_32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

template <bool kSigned>
__device__ __forceinline__ float tree_add(float a, float b) {
  // Sums of values that are each +0 or >= 2^-126 never land in the
  // subnormal range, so the flush is only needed when signs can differ.
  return kSigned ? fadd(a, b) : (a + b);
}

template <bool kSigned>
__device__ __forceinline__ float wave_tree(float v) {
  v = tree_add<kSigned>(v, dpp_xor1(v));
  v = tree_add<kSigned>(v, dpp_xor2(v));
  v = tree_add<kSigned>(v, dpp_half_mirror(v));
  v = tree_add<kSigned>(v, dpp_mirror(v));
  // binary32 addition is commutative bit for bit: lo + hi is each lane's
  // value plus its partner's
  LanePair p = lanes_16(v);
  v = tree_add<kSigned>(p.lo, p.hi);
  p = lanes_32(v);
  v = tree_add<kSigned>(p.lo, p.hi);
  return v;
}

// Tree over the first `w` lanes only (w a power of two <= 64): lanes in each
// aligned group of w end up holding that group's node.
template <bool kSigned>
__device__ __forceinline__ float wave_tree_partial(float v, int w) {
  if (w >= 2) v = tree_add<kSigned>(v, dpp_xor1(v));
  if (w >= 4) v = tree_add<kSigned>(v, dpp_xor2(v));
  if (w >= 8) v = tree_add<kSigned>(v, dpp_half_mirror(v));
  if (w >= 16) v = tree_add<kSigned>(v, dpp_mirror(v));
  if (w >= 32) {
    const LanePair p = lanes_16(v);
    v = tree_add<kSigned>(p.lo, p.hi);
  }
  if (w >= 64) {
    const LanePair p = lanes_32(v);
    v = tree_add<kSigned>(p.lo, p.hi);
  }
  return v;
}

// In-register tree over a[0..N), N a power of two; a is destroyed.
template <bool kSigned, int N>
__device__ __forceinline__ float reg_tree(float* a) {
#pragma unroll
  for (int w = N; w > 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w / 2; ++i) a[i] = tree_add<kSigned>(a[2 * i], a[2 * i + 1]);
  }
  return a[0];
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, dpp_half_mirror(v));
  v = fmaxf(v, dpp_mirror(v));
  LanePair p = lanes_16(v);
  v = fmaxf(p.lo, p.hi);
  p = lanes_32(v);
  v = fmaxf(p.lo, p.hi);
  return v;
}

// ---- 16-byte vectors -------------------------------------------------------
struct alignas(16) u32x4 { uint32_t x, y, z, w; };

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// DAZ of two bf16 values in one 32-bit word, on 16-bit halves: a half
// whose exponent field is zero keeps only its sign.  The exponent field is
// masked out, a packed minimum with 0x7f gives 0x7f in the halves whose
// exponent is nonzero and 0 in the others, and the mantissa bits of the
// latter are cleared (with the xor, one v_bitop3_b32).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_daz(uint32_t w) {
  const u16x2_t e = __builtin_bit_cast(u16x2_t, w & 0x7f807f80u);
  const u16x2_t m = __builtin_elementwise_min(e, u16x2_t{0x7f, 0x7f});
  return w & ~(__builtin_bit_cast(uint32_t, m) ^ 0x007f007fu);
}

// Unpack 16 bytes of bf16 (8 values) or fp32 (4 values) into floats (DAZ).
// bf16 widening is exact: the DAZ-ed halves shifted into the high bits.
__device__ __forceinline__ void unpack_bf16x8(u32x4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = bf16x2_daz(w[i]);
    f[2 * i] = __uint_as_float(u << 16);
    f[2 * i + 1] = __uint_as_float(u & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack_f32x4(u32x4 v, float* f) {
  f[0] = flush(__uint_as_float(v.x));
  f[1] = flush(__uint_as_float(v.y));
  f[2] = flush(__uint_as_float(v.z));
  f[3] = flush(__uint_as_float(v.w));
}

// Element type traits: values per 16-byte vector.
// Walsh-Hadamard butterflies over aligned blocks of B consecutive values
// (Sylvester order, unnormalised), stage order h = 1, 2, ..., B/2:
// (v_j, v_j+h) <- (fl(v_j + v_j+h), fl(v_j - v_j+h)).  Each lane holds P
// consecutive values; a block spans B / P consecutive lanes when B > P,
// else it sits inside the lane.  Every lane of the wave must call this.
template <int P, int B>
__device__ __forceinline__ void wht_block(float* f, int lane) {
#pragma unroll
  for (int h = 1; h < B; h *= 2) {
    if (h < P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        if ((j % (2 * h)) < h) {
          const float x0 = f[j], x1 = f[j + h];
          f[j] = fadd(x0, x1);
          f[j + h] = fsub(x0, x1);
        }
      }
    } else {
      const int dl = h / P;  // the partner lane holds the same j of the other half
      // the lower lane keeps fl(own + other); the upper lane keeps
      // fl(other - own), which IEEE defines as fl(other + (-own)): one add
      // with the sign of `own` flipped in the upper lane
      const uint32_t sgn = (lane & dl) ? 0x80000000u : 0u;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const float o = __shfl_xor(f[j], dl);
        f[j] = fadd(o, __uint_as_float(__float_as_uint(f[j]) ^ sgn));
      }
    }
  }
}

// ---- speculative unflushed evaluation ----------------------------------------
// A result that is not subnormal is left unchanged by the flush, so a run of
// operations evaluated without flushes equals the flushed evaluation
// whenever no input and no intermediate result is subnormal.  Kernels run
// that fast form, collect in `bad` the lanes where a value was subnormal
// (a compare into a lane mask, OR-ed on the scalar unit), and redo the
// whole wave's work with the flushes when the mask is not empty.
__device__ __forceinline__ uint64_t sub_mask(float v) {
  // one compare straight into a scalar lane mask (class bits 4 and 7:
  // -subnormal, +subnormal)
  uint64_t m;
  asm("v_cmp_class_f32_e64 %0, %1, %2" : "=s"(m) : "v"(v), "v"(0x090));
  return m;
}

// The butterflies of wht_block without flushes; subnormal results are
// recorded in `bad`.
template <int P, int B>
__device__ __forceinline__ void wht_block_fast(float* f, int lane, uint64_t& bad) {
#pragma unroll
  for (int h = 1; h < B; h *= 2) {
    if (h < P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        if ((j % (2 * h)) < h) {
          const float x0 = f[j], x1 = f[j + h];
          f[j] = x0 + x1;
          f[j + h] = x0 - x1;
          bad |= sub_mask(f[j]) | sub_mask(f[j + h]);
        }
      }
    } else {
      const int dl = h / P;
      const uint32_t sgn = (lane & dl) ? 0x80000000u : 0u;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const float o = __shfl_xor(f[j], dl);
        f[j] = o + __uint_as_float(__float_as_uint(f[j]) ^ sgn);
        bad |= sub_mask(f[j]);
      }
    }
  }
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;
  __device__ static void unpack(u32x4 v, float* f) { unpack_f32x4(v, f); }
  __device__ static float load1(const float* p, int64_t i) { return flush(p[i]); }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPerVec = 8;
  __device__ static void unpack(u32x4 v, float* f) { unpack_bf16x8(v, f); }
  __device__ static float load1(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
};

// raw 16-byte vectors -> floats without the DAZ flush (bf16 widened by a
// shift); subnormal inputs are recorded in `bad`
template <typename T>
__device__ __forceinline__ void widen_raw(u32x4 v, float* f, uint64_t& bad) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if (Elem<T>::kPerVec == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
#pragma unroll
  for (int e = 0; e < Elem<T>::kPerVec; ++e) bad |= sub_mask(f[e]);
}

// ---- explicit waits on the memory counters ----------------------------------
// gfx9 s_waitcnt immediate: vmcnt in bits [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8]; a field at its maximum does not wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}
// wait until at most n vector memory operations are outstanding; n is
// clamped to [0, MAXN] (callers pass counts that never exceed MAXN)
template <int MAXN>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (MAXN == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= MAXN) wait_vmcnt<MAXN>();
    else wait_vmcnt_upto<MAXN - 1>(n);
  }
}

// col mod cols, with a mask when cols is a power of two
__device__ __forceinline__ int64_t col_of(int64_t i, int64_t cols) {
  return (cols & (cols - 1)) == 0 ? (i & (cols - 1)) : i % cols;
}

__device__ __forceinline__ void set_flag(int32_t* flags, int32_t bit) {
  if (flags) atomicOr(flags, bit);
}

}  // namespace brq
