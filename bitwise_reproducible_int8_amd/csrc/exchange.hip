// exchange.hip -- the arithmetic of the deterministic data-parallel gradient
// exchange (Open-1B report, App. A "Deterministic Gradient Reduction"),
// for contributions resident on one device.
//
// Three levels reduce one step's gradient, each elementwise:
//   - microbatches of a rank: a running sum in microbatch order;
//   - shards of a node (App. A.2, the sum after the all-to-all of the
//     deterministic reduce-scatter): a running sum over shards 0 .. S-1 in
//     ascending order, finalised once per replica;
//   - replicas (App. A.1, the recursive-doubling all-reduce that TreeFold
//     replays): the binary-carry fold, lower replica on the left, and the
//     entries left for a count that is not a power of two combined smallest
//     block first.
// Each level's average is a multiply by the binary32 reciprocal of its count
// (App. A.3).  Every operation is one rounded binary32 operation, inputs
// read with DAZ and results flushed.
//
// The contributions arrive in mesh order (replica-major, then shard, then
// microbatch).  Each lane owns four consecutive elements and walks the
// contributions in that order with four 16-byte loads in flight; the level
// counters are wave-uniform, so the branches are scalar.  The fold keeps one
// register slot per level: pushing replica r merges with the slots of r's
// trailing one bits, exactly the stack that binary counting leaves.  The
// kernel is bound by HBM reads: (P + 1) * 4 bytes per element for P
// contributions.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

constexpr int kLevels = 7;  // 64 replicas need levels 0..6

struct PartPtrs {
  const float* p[BRQ_DP_MAX_PARTS];
};

struct F4 {
  float v[4];
};
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ F4 load4(const float* base, int64_t i0, int64_t n) {
  F4 r;
  if (i0 + 4 <= n) {
    const u32x4 w = ld16(base + i0);
    unpack_f32x4(w, r.v);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) r.v[e] = i0 + e < n ? flush(base[i0 + e]) : 0.0f;
  }
  return r;
}

__device__ __forceinline__ F4 add4(const F4& a, const F4& b) {
  F4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r.v[e] = fadd(a.v[e], b.v[e]);
  return r;
}

__device__ __forceinline__ F4 mul4(const F4& a, float c) {
  F4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r.v[e] = fmul(a.v[e], c);
  return r;
}

__global__ __launch_bounds__(256) void k_dp_reduce(PartPtrs parts, int R, int S, int A,
                                                   int64_t n, int average, float inv_a,
                                                   float inv_s, float inv_r,
                                                   float* __restrict__ out,
                                                   int32_t* dflags) {
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= n) return;
  const int P = R * S * A;

  // four contributions in flight ahead of the one being added
  F4 q0 = load4(parts.p[0], i0, n);
  F4 q1 = P > 1 ? load4(parts.p[1], i0, n) : q0;
  F4 q2 = P > 2 ? load4(parts.p[2], i0, n) : q0;
  F4 q3 = P > 3 ? load4(parts.p[3], i0, n) : q0;

  F4 acc_a = q0, inner = q0;
  F4 slot[kLevels];
#pragma unroll
  for (int l = 0; l < kLevels; ++l) slot[l] = q0;

  int a = 0, s = 0, r = 0;
  for (int j = 0; j < P; ++j) {
    const F4 cur = q0;
    q0 = q1;
    q1 = q2;
    q2 = q3;
    if (j + 4 < P) q3 = load4(parts.p[j + 4], i0, n);

    acc_a = a == 0 ? cur : add4(acc_a, cur);  // microbatch running sum
    if (++a < A) continue;
    a = 0;
    F4 g = average ? mul4(acc_a, inv_a) : acc_a;
    inner = s == 0 ? g : add4(inner, g);  // ascending shard sum
    if (++s < S) continue;
    s = 0;
    F4 e = average ? mul4(inner, inv_s) : inner;
    // push replica r: merge with the slots of r's trailing one bits (the
    // stack entries, which hold the lower replicas, on the left), then
    // store at the level above them
    const int t = __builtin_ctz(~(unsigned)r);
#pragma unroll
    for (int l = 0; l < kLevels; ++l) {
      if (l < t) e = add4(slot[l], e);
      if (l == t) slot[l] = e;
    }
    ++r;
  }

  // Result: the entries at the set bits of R, lowest level first
  F4 res = q0;
  bool have = false;
#pragma unroll
  for (int l = 0; l < kLevels; ++l) {
    if ((R >> l) & 1) {
      res = have ? add4(slot[l], res) : slot[l];
      have = true;
    }
  }
  if (average) res = mul4(res, inv_r);

  bool bad = false;
#pragma unroll
  for (int e = 0; e < 4; ++e) bad |= (i0 + e < n) && !__builtin_isfinite(res.v[e]);
  if (i0 + 4 <= n) {
    __builtin_nontemporal_store(f32x4_t{res.v[0], res.v[1], res.v[2], res.v[3]},
                                reinterpret_cast<f32x4_t*>(out + i0));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i0 + e < n) out[i0 + e] = res.v[e];
  }
  if (bad) set_flag(dflags, BRQ_FLAG_NONFINITE);
}

// binary32 reciprocal of a count on the host: one correctly rounded divide
// (a count <= 64 is exact in binary32, and its reciprocal is normal)
float host_reciprocal(int k) { return 1.0f / (float)k; }

}  // namespace

hipError_t dp_reduce(const float* const* parts, int R, int S, int A, int64_t n, int average,
                     float* out, int32_t* dflags, hipStream_t st) {
  if (n == 0) return hipSuccess;
  PartPtrs pp{};
  const int P = R * S * A;
  for (int j = 0; j < P; ++j) pp.p[j] = parts[j];
  const int64_t threads = (n + 3) / 4;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(k_dp_reduce, dim3((unsigned)blocks), dim3(256), 0, st, pp, R, S, A, n,
                     average, host_reciprocal(A), host_reciprocal(S), host_reciprocal(R), out,
                     dflags);
  return hipGetLastError();
}

}  // namespace brq
