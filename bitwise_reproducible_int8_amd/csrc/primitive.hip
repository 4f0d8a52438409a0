// primitive.hip -- the device's binary32 primitives on any range of inputs,
// for checking them against another machine's (Open-1B report, §2 "The same
// operation compiles to different instructions": a division or square root
// may lower to an approximation on one backend and to the correctly rounded
// operation on another; §2.1 Table 1: subnormals flushed everywhere).
//
// Input i of a sweep is the binary32 bit pattern first + i (mod 2^32).  Each
// primitive applies exactly the helpers the kernels use (device.hpp), so a
// sweep over all 2^32 patterns compares what the kernels execute with the
// host's correctly rounded operations.  Four inputs per lane, 16-byte
// stores; bound by the output writes.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

__device__ __forceinline__ uint32_t apply(int prim, uint32_t bits) {
  const float x = __uint_as_float(bits);
  switch (prim) {
    case BRQ_PRIM_SQRT: return __float_as_uint(fl_sqrt(flush(x)));
    case BRQ_PRIM_RCP: return __float_as_uint(fl_div(1.0f, flush(x)));
    case BRQ_PRIM_RSQRT: return __float_as_uint(fl_div(1.0f, fl_sqrt(flush(x))));
    case BRQ_PRIM_BF16_CVT: return pack2_bf16(x, 0.0f) & 0xffffu;
    default: return f32_to_bf16(x);  // BRQ_PRIM_BF16_INT
  }
}

template <int PRIM>
__global__ __launch_bounds__(256) void k_primitive(uint32_t first, int64_t count,
                                                   uint32_t* __restrict__ out) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= count) return;
  uint32_t r[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = apply(PRIM, first + (uint32_t)(i0 + e));
  if (i0 + 4 <= count) {
    st16(out + i0, u32x4{r[0], r[1], r[2], r[3]});
  } else {
    for (int e = 0; e < 4; ++e)
      if (i0 + e < count) out[i0 + e] = r[e];
  }
}

}  // namespace

hipError_t fp32_primitive(int prim, uint32_t first, int64_t count, uint32_t* out, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const int64_t blocks = ((count + 3) / 4 + 255) / 256;
  const dim3 g((unsigned)blocks), b(256);
  switch (prim) {
    case BRQ_PRIM_SQRT: hipLaunchKernelGGL(k_primitive<BRQ_PRIM_SQRT>, g, b, 0, s, first, count, out); break;
    case BRQ_PRIM_RCP: hipLaunchKernelGGL(k_primitive<BRQ_PRIM_RCP>, g, b, 0, s, first, count, out); break;
    case BRQ_PRIM_RSQRT: hipLaunchKernelGGL(k_primitive<BRQ_PRIM_RSQRT>, g, b, 0, s, first, count, out); break;
    case BRQ_PRIM_BF16_CVT: hipLaunchKernelGGL(k_primitive<BRQ_PRIM_BF16_CVT>, g, b, 0, s, first, count, out); break;
    default: hipLaunchKernelGGL(k_primitive<BRQ_PRIM_BF16_INT>, g, b, 0, s, first, count, out); break;
  }
  return hipGetLastError();
}

}  // namespace brq
