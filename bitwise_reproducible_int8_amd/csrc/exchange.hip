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
// microbatch).  Each lane owns kGroups groups of four consecutive elements,
// the groups 1024 elements apart, so every load instruction of a wave reads
// one contiguous kilobyte; loads are nontemporal (each value is read once)
// and two contributions are loaded ahead of their adds.  More groups per
// lane measured no faster and cost registers that the fold needs.  The
// level counters are uniform across the grid, so every branch on them is
// scalar, and each level starts from its first term rather than from a
// select.  The fold keeps one register slot per level (LV levels hold up to
// 2^LV - 1 replicas): pushing replica r merges the slots of r's trailing one
// bits, exactly the stack that binary counting leaves.  A multiply by the
// reciprocal of a count of one is the identity on flushed values and is
// skipped.  The kernel reads (P + 1) * 4 bytes per element for P
// contributions and is bound by HBM.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

constexpr int kLanes = 256;
constexpr int kGroups = 1;  // groups of four elements per lane
constexpr int kStride = kLanes * 4;  // elements between a lane's groups

struct PartPtrs {
  const float* p[BRQ_DP_MAX_PARTS];
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int G>
struct Vec {
  float v[4 * G];
};

// Contribution `p` at the lane's elements; EDGE: the work-group straddles n
// (elements at or beyond n read as 0 and are never stored).
template <int G, bool EDGE>
__device__ __forceinline__ Vec<G> vload(const float* p, int64_t i0, int64_t n) {
  Vec<G> r;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t i = i0 + (int64_t)g * kStride;
    if (!EDGE) {
      // each value is read once: a nontemporal load
      const f32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + i));
      const u32x4 u{__float_as_uint(w[0]), __float_as_uint(w[1]), __float_as_uint(w[2]),
                    __float_as_uint(w[3])};
      unpack_f32x4(u, r.v + 4 * g);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) r.v[4 * g + e] = i + e < n ? flush(p[i + e]) : 0.0f;
    }
  }
  return r;
}

template <int G>
__device__ __forceinline__ Vec<G> vadd(const Vec<G>& a, const Vec<G>& b) {
  Vec<G> r;
#pragma unroll
  for (int k = 0; k < 4 * G; ++k) r.v[k] = fadd(a.v[k], b.v[k]);
  return r;
}

template <int G>
__device__ __forceinline__ Vec<G> vmul(const Vec<G>& a, float c) {
  Vec<G> r;
#pragma unroll
  for (int k = 0; k < 4 * G; ++k) r.v[k] = fmul(a.v[k], c);
  return r;
}

// Running sum of contributions j .. j + count - 1, left to right.
template <int G, bool EDGE>
__device__ __forceinline__ Vec<G> run_sum(const PartPtrs& parts, int j, int count, int64_t i0,
                                          int64_t n) {
  Vec<G> acc = vload<G, EDGE>(parts.p[j], i0, n);
  int k = 1;
  for (; k + 1 < count; k += 2) {
    const Vec<G> x = vload<G, EDGE>(parts.p[j + k], i0, n);
    const Vec<G> y = vload<G, EDGE>(parts.p[j + k + 1], i0, n);
    acc = vadd(acc, x);
    acc = vadd(acc, y);
  }
  if (k < count) acc = vadd(acc, vload<G, EDGE>(parts.p[j + k], i0, n));
  return acc;
}

// Push replica r's value e: with t = the number of trailing one bits of r,
// merge the slots below level t into it (lower replicas on the left) and
// keep the sum at level t.
template <int G, int LV>
__device__ __forceinline__ void push(Vec<G> (&slot)[LV], Vec<G> e, int t) {
#pragma unroll
  for (int l = 0; l < LV; ++l) {
    if (l == t) slot[l] = e;
    if (l < t) e = vadd(slot[l], e);
  }
}

template <int G, int LV, bool EDGE>
__device__ __forceinline__ void reduce_lane(const PartPtrs& parts, int R, int S, int A,
                                            int64_t i0, int64_t n, int average, float inv_a,
                                            float inv_s, float inv_r, float* out,
                                            int32_t* dflags) {
  const bool avg_a = average && A > 1, avg_s = average && S > 1, avg_r = average && R > 1;
  Vec<G> slot[LV];
#pragma unroll
  for (int l = 0; l < LV; ++l)
#pragma unroll
    for (int k = 0; k < 4 * G; ++k) slot[l].v[k] = 0.0f;
  int j = 0;
  for (int r = 0; r < R; ++r) {
    Vec<G> e;
    if (A == 1) {
      e = run_sum<G, EDGE>(parts, j, S, i0, n);  // ascending shard sum
      j += S;
    } else {
      e = run_sum<G, EDGE>(parts, j, A, i0, n);  // microbatches of shard 0
      j += A;
      if (avg_a) e = vmul(e, inv_a);
      for (int s = 1; s < S; ++s) {
        Vec<G> g = run_sum<G, EDGE>(parts, j, A, i0, n);
        j += A;
        if (avg_a) g = vmul(g, inv_a);
        e = vadd(e, g);
      }
    }
    if (avg_s) e = vmul(e, inv_s);
    push(slot, e, __builtin_ctz(~(unsigned)r));
  }

  // Result: the entries at the set bits of R, lowest level first
  Vec<G> res = slot[0];
  bool have = false;
#pragma unroll
  for (int l = 0; l < LV; ++l) {
    if ((R >> l) & 1) {
      res = have ? vadd(slot[l], res) : slot[l];
      have = true;
    }
  }
  if (avg_r) res = vmul(res, inv_r);

  bool bad = false;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t i = i0 + (int64_t)g * kStride;
    float* v = res.v + 4 * g;
    if (average) {
      // a multiply by one skipped above would have quieted a lone
      // signalling NaN; every other value is unchanged by this
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_canonicalizef(v[e]);
    }
    if (!EDGE) {
#pragma unroll
      for (int e = 0; e < 4; ++e) bad |= !__builtin_isfinite(v[e]);
      __builtin_nontemporal_store(f32x4_t{v[0], v[1], v[2], v[3]},
                                  reinterpret_cast<f32x4_t*>(out + i));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (i + e < n) {
          bad |= !__builtin_isfinite(v[e]);
          out[i + e] = v[e];
        }
      }
    }
  }
  if (bad) set_flag(dflags, BRQ_FLAG_NONFINITE);
}

template <int G, int LV>
__global__ __launch_bounds__(kLanes) void k_dp_reduce(PartPtrs parts, int R, int S, int A,
                                                      int64_t n, int average, float inv_a,
                                                      float inv_s, float inv_r, float* out,
                                                      int32_t* dflags) {
  const int64_t base = (int64_t)blockIdx.x * (G * kStride);
  const int64_t i0 = base + (int64_t)threadIdx.x * 4;
  if (base + G * kStride <= n)
    reduce_lane<G, LV, false>(parts, R, S, A, i0, n, average, inv_a, inv_s, inv_r, out, dflags);
  else
    reduce_lane<G, LV, true>(parts, R, S, A, i0, n, average, inv_a, inv_s, inv_r, out, dflags);
}

// binary32 reciprocal of a count on the host: one correctly rounded divide
// (a count <= 64 is exact in binary32, and its reciprocal is normal)
float host_reciprocal(int k) { return 1.0f / (float)k; }

template <int G, int LV>
void launch(const PartPtrs& pp, int R, int S, int A, int64_t n, int average, float* out,
            int32_t* dflags, hipStream_t st) {
  const int64_t blocks = (n + G * kStride - 1) / (G * kStride);
  hipLaunchKernelGGL((k_dp_reduce<G, LV>), dim3((unsigned)blocks), dim3(kLanes), 0, st, pp, R,
                     S, A, n, average, host_reciprocal(A), host_reciprocal(S),
                     host_reciprocal(R), out, dflags);
}

}  // namespace

hipError_t dp_reduce(const float* const* parts, int R, int S, int A, int64_t n, int average,
                     float* out, int32_t* dflags, hipStream_t st) {
  if (n == 0) return hipSuccess;
  PartPtrs pp{};
  const int P = R * S * A;
  for (int j = 0; j < P; ++j) pp.p[j] = parts[j];
  // levels of the fold: floor(log2 R) + 1
  constexpr int G = kGroups;
  if (R == 1) launch<G, 1>(pp, R, S, A, n, average, out, dflags, st);
  else if (R < 4) launch<G, 2>(pp, R, S, A, n, average, out, dflags, st);
  else if (R < 8) launch<G, 3>(pp, R, S, A, n, average, out, dflags, st);
  else if (R < 16) launch<G, 4>(pp, R, S, A, n, average, out, dflags, st);
  else if (R < 32) launch<G, 5>(pp, R, S, A, n, average, out, dflags, st);
  else if (R < 64) launch<G, 6>(pp, R, S, A, n, average, out, dflags, st);
  else launch<G, 7>(pp, R, S, A, n, average, out, dflags, st);
  return hipGetLastError();
}

}  // namespace brq
