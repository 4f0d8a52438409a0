// optim.hip -- the optimizer step that consumes the layer's gradients
// (Open-1B report §3.2 "Optimizer": AdamW with beta1 0.9, beta2 0.95, eps
// 1e-8 through a reproducible fused kernel, decoupled weight decay 0.1 on
// the linear layers, gradients clipped to a global l2 norm of 1.0; §3.2
// "Optimizer-state precision": BF16 parameters and FP32 moments, widened,
// updated in FP32 and rounded to BF16 once per step; §3.4.2 "Gradient
// behavior, Clipping, and Spike Protocol": five optimizer steps skipped when
// the pre-clip norm exceeds 5).
//
// Every element is independent, so there is no order to fix beyond the
// operation sequence of one element (each operation one rounded, flushed
// binary32 operation):
//   g  = clip != 1 ? g * clip : g
//   m  = b1*m + (1-b1)*g            v = b2*v + (1-b2)*(g*g)
//   mh = m / bc1     vh = v / bc2   u = mh / (sqrt(vh) + eps)
//   p  = p - lr*(u + wd*p)
// Division and square root are the correctly rounded binary32 operations.
//
// The decision (skip window, clip scale) is one thread reading the device
// grad-norm, so the host never waits for it; the update reads the decision.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

__global__ void k_adamw_decide(const float* __restrict__ norm_in, float max_norm, float spike,
                               int skip_steps, int32_t* skip_state, float* ctl,
                               int32_t* dflags) {
  if (threadIdx.x != 0) return;
  const float norm = flush(norm_in[0]);
  const bool finite = __builtin_isfinite(norm);
  int32_t st = skip_state[0];
  if (!finite || norm > spike) st = skip_steps;
  float apply, clip;
  if (st > 0) {
    st -= 1;
    apply = 0.0f;
    clip = 0.0f;
  } else {
    apply = 1.0f;
    clip = norm > flush(max_norm) ? fl_div(flush(max_norm), norm) : 1.0f;
  }
  skip_state[0] = st;
  ctl[0] = apply;
  ctl[1] = clip;
  if (!finite) set_flag(dflags, BRQ_FLAG_NONFINITE);
}

struct Hp {
  float lr, beta1, beta2, eps, wd, bc1, bc2;
};

// Packing for the stores: bf16 rounds to nearest even once, fp32 as is.
__device__ __forceinline__ u32x4 pack8_bf16(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack2_bf16(f[2 * i], f[2 * i + 1]);
  return u32x4{w[0], w[1], w[2], w[3]};
}
__device__ __forceinline__ u32x4 pack4_f32(const float* f) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
               __float_as_uint(f[3])};
}
__device__ __forceinline__ void store1(uint16_t* p, int64_t i, float f) {
  p[i] = (uint16_t)f32_to_bf16(f);
}
__device__ __forceinline__ void store1(float* p, int64_t i, float f) { p[i] = f; }

// 8 consecutive elements per lane: one 16-byte vector of bf16, two of fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* p, int64_t i0, int64_t n, float* f) {
  if (i0 + 8 <= n) {
    if constexpr (Elem<T>::kPerVec == 8) {
      Elem<T>::unpack(ld16(p + i0), f);
    } else {
      Elem<T>::unpack(ld16(p + i0), f);
      Elem<T>::unpack(ld16(p + i0 + 4), f + 4);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = i0 + e < n ? Elem<T>::load1(p, i0 + e) : 0.0f;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, int64_t i0, int64_t n, const float* f) {
  if (i0 + 8 <= n) {
    if constexpr (Elem<T>::kPerVec == 8) {
      st16(p + i0, pack8_bf16(f));
    } else {
      st16(p + i0, pack4_f32(f));
      st16(p + i0 + 4, pack4_f32(f + 4));
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (i0 + e < n) store1(p, i0 + e, f[e]);
  }
}

template <typename TP, typename TG>
__global__ __launch_bounds__(256) void k_adamw_step(TP* __restrict__ param,
                                                    const TG* __restrict__ grad,
                                                    float* __restrict__ m, float* __restrict__ v,
                                                    int64_t n, Hp hp,
                                                    const float* __restrict__ ctl) {
  if (ctl[0] == 0.0f) return;  // a skipped step changes nothing
  const float clip = ctl[1];
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= n) return;
  const float omb1 = fsub(1.0f, hp.beta1), omb2 = fsub(1.0f, hp.beta2);
  float p[8], g[8], mm[8], vv[8];
  load8<TP>(param, i0, n, p);
  load8<TG>(grad, i0, n, g);
  load8<float>(m, i0, n, mm);
  load8<float>(v, i0, n, vv);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float ge = g[e];
    if (clip != 1.0f) ge = fmul(ge, clip);
    const float mi = fadd(fmul(hp.beta1, mm[e]), fmul(omb1, ge));
    const float vi = fadd(fmul(hp.beta2, vv[e]), fmul(omb2, fmul(ge, ge)));
    const float mh = fl_div(mi, hp.bc1);
    const float vh = fl_div(vi, hp.bc2);
    const float u = fl_div(mh, fadd(fl_sqrt(vh), hp.eps));
    p[e] = fsub(p[e], fmul(hp.lr, fadd(u, fmul(hp.wd, p[e]))));
    mm[e] = mi;
    vv[e] = vi;
  }
  store8<TP>(param, i0, n, p);
  store8<float>(m, i0, n, mm);
  store8<float>(v, i0, n, vv);
}

template <typename TP, typename TG>
hipError_t launch_step(void* param, const void* grad, float* m, float* v, int64_t n, Hp hp,
                       const float* ctl, hipStream_t s) {
  const int64_t blocks = (n + 8 * 256 - 1) / (8 * 256);
  hipLaunchKernelGGL((k_adamw_step<TP, TG>), dim3((unsigned)blocks), dim3(256), 0, s,
                     (TP*)param, (const TG*)grad, m, v, n, hp, ctl);
  return hipGetLastError();
}

}  // namespace

hipError_t adamw_decide(const float* norm, float max_norm, float spike, int skip_steps,
                        int32_t* skip_state, float* ctl, int32_t* dflags, hipStream_t s) {
  hipLaunchKernelGGL(k_adamw_decide, dim3(1), dim3(64), 0, s, norm, max_norm, spike, skip_steps,
                     skip_state, ctl, dflags);
  return hipGetLastError();
}

hipError_t adamw_step(void* param, int pdtype, const void* grad, int gdtype, float* m, float* v,
                      int64_t n, const brq_adamw_hparams& h, const float* ctl, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const Hp hp{h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.bias_correction1,
              h.bias_correction2};
  if (pdtype == BRQ_BF16 && gdtype == BRQ_F32)
    return launch_step<uint16_t, float>(param, grad, m, v, n, hp, ctl, s);
  if (pdtype == BRQ_BF16) return launch_step<uint16_t, uint16_t>(param, grad, m, v, n, hp, ctl, s);
  if (gdtype == BRQ_F32) return launch_step<float, float>(param, grad, m, v, n, hp, ctl, s);
  return launch_step<float, uint16_t>(param, grad, m, v, n, hp, ctl, s);
}

}  // namespace brq
