// hash.hip -- on-device canonical state hash.  The Open-1B report (§5
// "Runtime overhead", App. B) hashes the training state every step on the
// host at about 6 s per step and names on-device hashing as the fix; this
// is that hash on the GPU: SHA-256 (FIPS 180-4) Merkle trees over the raw
// tensor bytes, 4096-byte leaves, 128 digests per interior node, a typed
// header per tensor, and one digest over all tensor digests in call order.
//
// The work is integer ALU (about 24 VALU operations per hashed byte), so
// the kernels are built to keep every SIMD busy:
//   - one launch hashes every full 4096-byte slice of up to kBatch buffers
//     (all tensors' leaves together, then each Merkle level of all tensors
//     together), one lane per slice; a second, one-wave launch takes each
//     buffer's shorter last slice;
//   - a full slice streams its 64 blocks (other waves hide the load
//     latency), and its 65th (padding) block is a constant;
//   - the round function is written in the shapes gfx950 has single
//     instructions for: rotate (v_alignbit_b32), three-way xor, choose and
//     majority (v_bitop3_b32), three-way add (v_add3_u32).
#include <limits.h>
#include <string.h>

#include "device.hpp"
#include "internal.hpp"

namespace brq {

namespace {

constexpr int kLeaf = 4096;     // bytes per leaf (and per interior node's input)
constexpr int kFan = 128;       // digests per interior node
constexpr int kBatch = 32;      // buffers per slice launch
constexpr int kHdrBatch = 32;   // tensor headers per header launch
constexpr int kHdrMax = 336;    // header bytes: 4+1+1+8*8+2+255 = 327
constexpr int kHdrBlob = 2048;  // header bytes per launch, packed back to back

__constant__ uint32_t kSha256K[64] = {
    0x428a2f98u, 0x71374491u, 0xb5c0fbcfu, 0xe9b5dba5u, 0x3956c25bu, 0x59f111f1u, 0x923f82a4u,
    0xab1c5ed5u, 0xd807aa98u, 0x12835b01u, 0x243185beu, 0x550c7dc3u, 0x72be5d74u, 0x80deb1feu,
    0x9bdc06a7u, 0xc19bf174u, 0xe49b69c1u, 0xefbe4786u, 0x0fc19dc6u, 0x240ca1ccu, 0x2de92c6fu,
    0x4a7484aau, 0x5cb0a9dcu, 0x76f988dau, 0x983e5152u, 0xa831c66du, 0xb00327c8u, 0xbf597fc7u,
    0xc6e00bf3u, 0xd5a79147u, 0x06ca6351u, 0x14292967u, 0x27b70a85u, 0x2e1b2138u, 0x4d2c6dfcu,
    0x53380d13u, 0x650a7354u, 0x766a0abbu, 0x81c2c92eu, 0x92722c85u, 0xa2bfe8a1u, 0xa81a664bu,
    0xc24b8b70u, 0xc76c51a3u, 0xd192e819u, 0xd6990624u, 0xf40e3585u, 0x106aa070u, 0x19a4c116u,
    0x1e376c08u, 0x2748774cu, 0x34b0bcb5u, 0x391c0cb3u, 0x4ed8aa4au, 0x5b9cca4fu, 0x682e6ff3u,
    0x748f82eeu, 0x78a5636fu, 0x84c87814u, 0x8cc70208u, 0x90befffau, 0xa4506cebu, 0xbef9a3f7u,
    0xc67178f2u};

__device__ __forceinline__ uint32_t rotr(uint32_t x, int n) {
  return __builtin_amdgcn_alignbit(x, x, n);
}
__device__ __forceinline__ uint32_t bswap(uint32_t x) { return __builtin_bswap32(x); }
// x ^ y ^ z in one v_bitop3_b32 (truth table 0x96, symmetric in its inputs)
__device__ __forceinline__ uint32_t xor3(uint32_t x, uint32_t y, uint32_t z) {
  return __builtin_amdgcn_bitop3_b32(x, y, z, 0x96);
}
// (m & x) | (~m & y) in one v_bitop3_b32: the truth table is indexed by
// (m << 2) | (x << 1) | y, so entries 1, 3 (y), 6, 7 (x) are set: 0xCA
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t x, uint32_t y) {
  return __builtin_amdgcn_bitop3_b32(m, x, y, 0xCA);
}

struct Sha {
  uint32_t h[8];
  __device__ __forceinline__ void init() {
    h[0] = 0x6a09e667u; h[1] = 0xbb67ae85u; h[2] = 0x3c6ef372u; h[3] = 0xa54ff53au;
    h[4] = 0x510e527fu; h[5] = 0x9b05688cu; h[6] = 0x1f83d9abu; h[7] = 0x5be0cd19u;
  }
  // One compression of 16 big-endian message words (FIPS 180-4 §6.2.2).
  __device__ __forceinline__ void block(const uint32_t* win) {
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = win[i];
    uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      uint32_t wt;
      if (t < 16) {
        wt = w[t];
      } else {
        const uint32_t w15 = w[(t - 15) & 15], w2 = w[(t - 2) & 15];
        const uint32_t s0 = xor3(rotr(w15, 7), rotr(w15, 18), w15 >> 3);
        const uint32_t s1 = xor3(rotr(w2, 17), rotr(w2, 19), w2 >> 10);
        wt = w[t & 15] + s0 + w[(t - 7) & 15] + s1;
        w[t & 15] = wt;
      }
      const uint32_t S1 = xor3(rotr(e, 6), rotr(e, 11), rotr(e, 25));
      const uint32_t t1 = hh + S1 + bitsel(e, f, g) + kSha256K[t] + wt;
      const uint32_t S0 = xor3(rotr(a, 2), rotr(a, 13), rotr(a, 22));
      // majority(a, b, c): one v_bitop3_b32, truth table 0xE8 (symmetric)
      const uint32_t mj = __builtin_amdgcn_bitop3_b32(a, b, c, 0xE8);
      hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + S0 + mj;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }
  __device__ __forceinline__ void store(uint8_t* out) const {
    st16(out, u32x4{bswap(h[0]), bswap(h[1]), bswap(h[2]), bswap(h[3])});
    st16(out + 16, u32x4{bswap(h[4]), bswap(h[5]), bswap(h[6]), bswap(h[7])});
  }
};

__device__ __forceinline__ void be_words(const u32x4* v, uint32_t* w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w[4 * i] = bswap(v[i].x);
    w[4 * i + 1] = bswap(v[i].y);
    w[4 * i + 2] = bswap(v[i].z);
    w[4 * i + 3] = bswap(v[i].w);
  }
}

// Tail of a message: `rem` (< 64) bytes at p, then 0x80, zero fill and the
// 64-bit big-endian bit length; one or two blocks.  Byte loads under their
// own predicates keep the block words at static register indices.
__device__ void sha_tail(Sha& st, const uint8_t* p, int rem, uint64_t total_len) {
  uint32_t w[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) w[i] = 0;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    uint32_t byte = i < rem ? (uint32_t)p[i] : (i == rem ? 0x80u : 0u);
    w[i >> 2] |= byte << (24 - 8 * (i & 3));
  }
  const uint64_t bits = total_len * 8;
  if (rem + 1 + 8 <= 64) {
    w[14] = (uint32_t)(bits >> 32);
    w[15] = (uint32_t)bits;
    st.block(w);
  } else {
    w[30] = (uint32_t)(bits >> 32);
    w[31] = (uint32_t)bits;
    st.block(w);
    st.block(w + 16);
  }
}

// Digest of len bytes at p (16-byte aligned): full blocks by 16-byte loads.
__device__ void sha256_bytes(const uint8_t* p, uint64_t len, uint8_t* out) {
  Sha st;
  st.init();
  const uint64_t full = len / 64;
  for (uint64_t i = 0; i < full; ++i) {
    const u32x4* q = reinterpret_cast<const u32x4*>(p + 64 * i);
    u32x4 v[4] = {q[0], q[1], q[2], q[3]};
    uint32_t w[16];
    be_words(v, w);
    st.block(w);
  }
  sha_tail(st, p + 64 * full, (int)(len - 64 * full), len);
  st.store(out);
}

// A full 4096-byte slice: 64 data blocks, then the constant padding block
// (0x80, zeros, bit length 32768).  Load latency is hidden by the other
// waves of the SIMD rather than by a prefetch that would cost 16 registers.
__device__ __forceinline__ void sha256_slice4096(const uint8_t* p, uint8_t* out) {
  Sha st;
  st.init();
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
#pragma unroll 1
  for (int i = 0; i < kLeaf / 64; ++i) {
    const u32x4 cur[4] = {q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]};
    uint32_t w[16];
    be_words(cur, w);
    st.block(w);
  }
  uint32_t pad[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) pad[i] = 0;
  pad[0] = 0x80000000u;
  pad[15] = (uint32_t)(kLeaf * 8);
  st.block(pad);
  st.store(out);
}

// Slices of up to kBatch buffers: buffer i has n_slices[i] = max(1,
// ceil(nbytes[i] / 4096)) slices, and slice j's digest goes to dst[i] +
// 32 j.  first[] holds the prefix sums of the slice counts.
struct SliceBatch {
  const uint8_t* src[kBatch];
  uint8_t* dst[kBatch];
  uint64_t nbytes[kBatch];
  uint64_t first[kBatch + 1];
  int n;
};

// Full 4096-byte slices, one lane each; a buffer's partial last slice (or
// the one empty slice of an empty buffer) is left to k_sha_partial.  Kept
// apart from the generic path so the 4 KiB loop needs few registers: six
// waves per SIMD is the most at which the loop keeps its state in registers
// (at eight the compiler spills the chaining value inside the block loop).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void k_sha_full(
    SliceBatch b) {
  const uint64_t g = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= b.first[b.n]) return;
  int i = 0;
  while (i + 1 < b.n && g >= b.first[i + 1]) ++i;
  const uint64_t j = g - b.first[i];
  const uint64_t off = j * kLeaf;
  if (b.nbytes[i] >= off + kLeaf) sha256_slice4096(b.src[i] + off, b.dst[i] + 32 * j);
}

// The last slice of each buffer when it is shorter than 4096 bytes.
__global__ __launch_bounds__(64) void k_sha_partial(SliceBatch b) {
  const int i = threadIdx.x;
  if (i >= b.n) return;
  const uint64_t nb = b.nbytes[i];
  if (nb != 0 && nb % kLeaf == 0) return;
  const uint64_t j = b.first[i + 1] - b.first[i] - 1;
  const uint64_t off = j * kLeaf;
  sha256_bytes(b.src[i] + off, nb - off, b.dst[i] + 32 * j);
}

// Tensor digests: SHA-256(header | root), one lane per tensor.
// Headers packed back to back in one blob (header k at bytes off[k] ..
// off[k] + len[k] - 1), so that a launch's kernel argument holds up to
// kHdrBatch of them.
struct HeaderBatch {
  uint8_t bytes[kHdrBlob];
  uint16_t off[kHdrBatch];
  uint16_t len[kHdrBatch];
  const uint8_t* root[kHdrBatch];
  uint8_t* out[kHdrBatch];
  int n;
};

__global__ __launch_bounds__(64) void k_sha_headers(HeaderBatch hb) {
  // lane i stages its header (out of the blob) and its tensor's root in
  // LDS and hashes that message
  static_assert(kHdrBatch <= 64, "one lane per header");
  __shared__ __attribute__((aligned(16))) uint8_t msg[kHdrBatch][kHdrMax + 32];
  const int i = threadIdx.x;
  if (i >= hb.n) return;
  const int n = hb.len[i];
  for (int k = 0; k < n; ++k) msg[i][k] = hb.bytes[hb.off[i] + k];
  const int len = n + 32;
  for (int k = 0; k < 32; ++k) msg[i][n + k] = hb.root[i][k];
  Sha st;
  st.init();
  int off = 0;
  for (; off + 64 <= len; off += 64) {
    uint32_t w[16];
    for (int q = 0; q < 16; ++q)
      w[q] = ((uint32_t)msg[i][off + 4 * q] << 24) | ((uint32_t)msg[i][off + 4 * q + 1] << 16) |
             ((uint32_t)msg[i][off + 4 * q + 2] << 8) | (uint32_t)msg[i][off + 4 * q + 3];
    st.block(w);
  }
  sha_tail(st, &msg[i][off], len - off, (uint64_t)len);
  st.store(hb.out[i]);
}

// State digest over n tensor digests (32 n bytes, 16-byte aligned).
__global__ void k_sha_state(const uint8_t* __restrict__ digests, int n, uint8_t* __restrict__ out) {
  sha256_bytes(digests, (uint64_t)n * 32, out);
}

uint64_t cdivu(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

uint64_t tensor_bytes(const brq_tensor_ref& t) {
  static const int esz[5] = {4, 2, 1, 4, 1};
  uint64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= (uint64_t)t.dims[i];
  return n * (uint64_t)esz[t.dtype];
}

// Digest counts of tensor i's levels: level 0 = leaves, then ceil(/128)
// until one remains.  Returns the number of levels.
int level_counts(uint64_t nbytes, uint64_t* cnt) {
  int L = 0;
  cnt[L++] = nbytes == 0 ? 1 : cdivu(nbytes, kLeaf);
  while (cnt[L - 1] > 1) {
    cnt[L] = cdivu(cnt[L - 1], kFan);
    ++L;
  }
  return L;
}

// Bytes of one tensor's digest region (every level, 256-byte aligned).
size_t tensor_region(uint64_t nbytes) {
  uint64_t cnt[40];
  int L = level_counts(nbytes, cnt);
  size_t s = 0;
  for (int l = 0; l < L; ++l) s += align256(32 * cnt[l]);
  return s;
}

hipError_t launch_slices(SliceBatch& b, hipStream_t s) {
  if (b.n == 0) return hipSuccess;
  const uint64_t total = b.first[b.n];
  hipLaunchKernelGGL(k_sha_full, dim3((unsigned)cdivu(total, 256)), dim3(256), 0, s, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_sha_partial, dim3(1), dim3(64), 0, s, b);
  b.n = 0;
  b.first[0] = 0;
  return hipGetLastError();
}

void add_slices(SliceBatch& b, const uint8_t* src, uint64_t nbytes, uint8_t* dst) {
  const uint64_t cnt = nbytes == 0 ? 1 : cdivu(nbytes, kLeaf);
  b.src[b.n] = src;
  b.dst[b.n] = dst;
  b.nbytes[b.n] = nbytes;
  b.first[b.n + 1] = b.first[b.n] + cnt;
  ++b.n;
}

}  // namespace

size_t hash_digests_ws(const brq_tensor_ref* t, int n) {
  size_t s = 256;
  for (int i = 0; i < n; ++i) s += tensor_region(tensor_bytes(t[i]));
  return s;
}

size_t hash_ws(const brq_tensor_ref* t, int n) {
  return align256(32 * (uint64_t)(n > 0 ? n : 1)) + hash_digests_ws(t, n);
}

namespace {

// Merkle levels l0 <= l < l1 of every tensor: level 0 hashes tensor bytes,
// level l > 0 the digests of level l - 1; tensors whose tree has ended drop
// out, and the pass stops when every tree has.
hipError_t hash_levels(const brq_tensor_ref* t, int n, void* ws, int l0, int l1, hipStream_t s) {
  uint8_t* base = (uint8_t*)ws;
  hipError_t e;
  SliceBatch b{};
  for (int l = l0; l < l1; ++l) {
    bool any = false;
    uint8_t* region = base;
    for (int i = 0; i < n; ++i) {
      const uint64_t nb = tensor_bytes(t[i]);
      uint64_t cnt[40];
      const int L = level_counts(nb, cnt);
      uint8_t* lv[40];
      uint8_t* r = region;
      for (int k = 0; k < L; ++k) {
        lv[k] = r;
        r += align256(32 * cnt[k]);
      }
      region = r;
      if (l >= L) continue;
      any = true;
      if (l == 0) add_slices(b, (const uint8_t*)t[i].data, nb, lv[0]);
      else add_slices(b, lv[l - 1], 32 * cnt[l - 1], lv[l]);
      if (b.n == kBatch && (e = launch_slices(b, s)) != hipSuccess) return e;
    }
    if ((e = launch_slices(b, s)) != hipSuccess) return e;
    if (!any) break;
  }
  return hipSuccess;
}

// Tensor digests SHA-256(header | root) once every tree is complete.
hipError_t hash_headers(const brq_tensor_ref* t, int n, uint8_t* tdig, void* ws, hipStream_t s) {
  uint8_t* base = (uint8_t*)ws;
  hipError_t e;
  HeaderBatch hb{};
  int used = 0;  // blob bytes taken by the batch
  uint8_t* region = base;
  for (int i = 0; i < n; ++i) {
    const uint64_t nb = tensor_bytes(t[i]);
    uint64_t cnt[40];
    const int L = level_counts(nb, cnt);
    uint8_t* r = region;
    uint8_t* root = r;
    for (int k = 0; k < L; ++k) {
      root = r;
      r += align256(32 * cnt[k]);
    }
    region = r;
    uint8_t h[kHdrMax];
    int o = 0;
    h[o++] = 'B'; h[o++] = 'R'; h[o++] = 'Q'; h[o++] = '1';
    h[o++] = (uint8_t)t[i].dtype;
    h[o++] = (uint8_t)t[i].ndim;
    for (int d = 0; d < t[i].ndim; ++d)
      for (int q = 0; q < 8; ++q) h[o++] = (uint8_t)((uint64_t)t[i].dims[d] >> (8 * q));
    size_t nl = 0;
    while (t[i].name && t[i].name[nl]) ++nl;
    h[o++] = (uint8_t)(nl & 0xff);
    h[o++] = (uint8_t)(nl >> 8);
    for (size_t c = 0; c < nl; ++c) h[o++] = (uint8_t)t[i].name[c];
    // a full batch or blob goes out first
    if (hb.n == kHdrBatch || used + o > kHdrBlob) {
      hipLaunchKernelGGL(k_sha_headers, dim3(1), dim3(64), 0, s, hb);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hb.n = 0;
      used = 0;
    }
    const int k = hb.n++;
    memcpy(hb.bytes + used, h, (size_t)o);
    hb.off[k] = (uint16_t)used;
    hb.len[k] = (uint16_t)o;
    hb.root[k] = root;
    hb.out[k] = tdig + 32 * i;
    used += o;
  }
  if (hb.n > 0) {
    hipLaunchKernelGGL(k_sha_headers, dim3(1), dim3(64), 0, s, hb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t hash_tensor_digests(const brq_tensor_ref* t, int n, uint8_t* tdig, void* ws,
                               hipStream_t s) {
  hipError_t e = hash_levels(t, n, ws, 0, INT_MAX, s);
  if (e != hipSuccess) return e;
  return hash_headers(t, n, tdig, ws, s);
}

// The leaf level alone: the only part that reads the tensors.
hipError_t hash_tensor_leaves(const brq_tensor_ref* t, int n, void* ws, hipStream_t s) {
  return hash_levels(t, n, ws, 0, 1, s);
}

// Every level above the leaves, then the tensor digests: reads only ws.
hipError_t hash_tensor_finish(const brq_tensor_ref* t, int n, uint8_t* tdig, void* ws,
                              hipStream_t s) {
  hipError_t e = hash_levels(t, n, ws, 1, INT_MAX, s);
  if (e != hipSuccess) return e;
  return hash_headers(t, n, tdig, ws, s);
}

hipError_t hash_combine(const uint8_t* tdig, int n, uint8_t* digest32, hipStream_t s) {
  hipLaunchKernelGGL(k_sha_state, dim3(1), dim3(1), 0, s, tdig, n, digest32);
  return hipGetLastError();
}

hipError_t hash_state(const brq_tensor_ref* t, int n, uint8_t* digest32, void* ws, hipStream_t s) {
  uint8_t* tdig = (uint8_t*)ws;
  void* rest = tdig + align256(32 * (uint64_t)(n > 0 ? n : 1));
  hipError_t e = hash_tensor_digests(t, n, tdig, rest, s);
  if (e != hipSuccess) return e;
  return hash_combine(tdig, n, digest32, s);
}

}  // namespace brq
