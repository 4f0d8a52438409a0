// hash.hip -- on-device canonical state hash.  The Open-1B report (§5
// "Runtime overhead", App. B) hashes the training state every step on the
// host at about 6 s per step and names on-device hashing as the fix; this
// is that hash on the GPU: SHA-256 (FIPS 180-4) Merkle trees over the raw
// tensor bytes, 4096-byte leaves, 128 digests per interior node, a typed
// header per tensor, and one digest over all tensor digests in call order.
//
// The leaf pass is integer ALU work: one lane per 4096-byte leaf runs 64 or
// 65 compressions with the message schedule in registers.
#include "device.hpp"
#include "internal.hpp"

namespace brq {

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

__device__ __forceinline__ uint32_t rotr32(uint32_t x, int n) {
  return __builtin_amdgcn_alignbit(x, x, n);
}
__device__ __forceinline__ uint32_t bswap32(uint32_t x) {
  return __builtin_bswap32(x);
}

struct Sha {
  uint32_t h[8];
  __device__ void init() {
    h[0] = 0x6a09e667u; h[1] = 0xbb67ae85u; h[2] = 0x3c6ef372u; h[3] = 0xa54ff53au;
    h[4] = 0x510e527fu; h[5] = 0x9b05688cu; h[6] = 0x1f83d9abu; h[7] = 0x5be0cd19u;
  }
  // One compression of 16 big-endian words.
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
        uint32_t w15 = w[(t - 15) & 15], w2 = w[(t - 2) & 15];
        uint32_t s0 = rotr32(w15, 7) ^ rotr32(w15, 18) ^ (w15 >> 3);
        uint32_t s1 = rotr32(w2, 17) ^ rotr32(w2, 19) ^ (w2 >> 10);
        wt = w[t & 15] + s0 + w[(t - 7) & 15] + s1;
        w[t & 15] = wt;
      }
      uint32_t S1 = rotr32(e, 6) ^ rotr32(e, 11) ^ rotr32(e, 25);
      uint32_t ch = (e & f) ^ (~e & g);
      uint32_t t1 = hh + S1 + ch + kSha256K[t] + wt;
      uint32_t S0 = rotr32(a, 2) ^ rotr32(a, 13) ^ rotr32(a, 22);
      uint32_t mj = (a & b) ^ (a & c) ^ (b & c);
      uint32_t t2 = S0 + mj;
      hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
    }
    h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
  }
  __device__ void store(uint8_t* out) const {
    u32x4 lo{bswap32(h[0]), bswap32(h[1]), bswap32(h[2]), bswap32(h[3])};
    u32x4 hi{bswap32(h[4]), bswap32(h[5]), bswap32(h[6]), bswap32(h[7])};
    st16(out, lo);
    st16(out + 16, hi);
  }
};

// Tail of a message: `rem` (< 64) bytes at p, then 0x80, zero fill and the
// 64-bit big-endian bit length; one or two blocks.  Byte loads only, each
// under its own predicate, so the block words keep static register indices.
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

// Digest of `len` bytes at p (p 16-byte aligned); full blocks use 16-byte
// loads, the tail byte loads.
__device__ void sha256_region(const uint8_t* p, uint64_t len, uint8_t* out) {
  Sha st;
  st.init();
  const uint64_t full = len / 64;
  for (uint64_t i = 0; i < full; ++i) {
    const uint8_t* q = p + 64 * i;
    u32x4 v0 = ld16(q), v1 = ld16(q + 16), v2 = ld16(q + 32), v3 = ld16(q + 48);
    uint32_t w[16] = {bswap32(v0.x), bswap32(v0.y), bswap32(v0.z), bswap32(v0.w),
                      bswap32(v1.x), bswap32(v1.y), bswap32(v1.z), bswap32(v1.w),
                      bswap32(v2.x), bswap32(v2.y), bswap32(v2.z), bswap32(v2.w),
                      bswap32(v3.x), bswap32(v3.y), bswap32(v3.z), bswap32(v3.w)};
    st.block(w);
  }
  sha_tail(st, p + 64 * full, (int)(len - 64 * full), len);
  st.store(out);
}

// One lane per leaf of `leaf` bytes (4096): digest i covers
// [i*leaf, min((i+1)*leaf, nbytes)).  An empty buffer has one empty leaf.
__global__ __launch_bounds__(64) void k_sha_leaves(const uint8_t* __restrict__ data, uint64_t nbytes,
                                                   uint64_t nleaves, uint8_t* __restrict__ out) {
  const uint64_t i = (uint64_t)blockIdx.x * 64 + threadIdx.x;
  if (i >= nleaves) return;
  const uint64_t off = i * 4096;
  const uint64_t len = nbytes > off ? (nbytes - off < 4096 ? nbytes - off : 4096) : 0;
  sha256_region(data + off, len, out + 32 * i);
}

// Tensor digest: header prefix (passed by value) followed by the root.
struct HeaderArg {
  uint8_t bytes[352];
  int len;
};

__global__ void k_sha_header(HeaderArg h, const uint8_t* __restrict__ root, uint8_t* __restrict__ out) {
  uint8_t msg[352 + 32];
  const int n = h.len;
  for (int i = 0; i < n; ++i) msg[i] = h.bytes[i];
  for (int i = 0; i < 32; ++i) msg[n + i] = root[i];
  const int len = n + 32;
  Sha st;
  st.init();
  int off = 0;
  for (; off + 64 <= len; off += 64) {
    uint32_t w[16];
    for (int j = 0; j < 16; ++j)
      w[j] = ((uint32_t)msg[off + 4 * j] << 24) | ((uint32_t)msg[off + 4 * j + 1] << 16) |
             ((uint32_t)msg[off + 4 * j + 2] << 8) | (uint32_t)msg[off + 4 * j + 3];
    st.block(w);
  }
  sha_tail(st, msg + off, len - off, (uint64_t)len);
  st.store(out);
}

// State digest over n tensor digests (32 n bytes, 16-byte aligned).
__global__ void k_sha_state(const uint8_t* __restrict__ digests, int n, uint8_t* __restrict__ out) {
  sha256_region(digests, (uint64_t)n * 32, out);
}

static uint64_t cdivu(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

static uint64_t tensor_bytes(const brq_tensor_ref& t) {
  static const int esz[5] = {4, 2, 1, 4, 1};
  uint64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= (uint64_t)t.dims[i];
  return n * (uint64_t)esz[t.dtype];
}

size_t hash_ws(const brq_tensor_ref* t, int n) {
  uint64_t maxleaf = 1;
  for (int i = 0; i < n; ++i) {
    uint64_t l = cdivu(tensor_bytes(t[i]), 4096);
    if (l > maxleaf) maxleaf = l;
  }
  return align256(32 * maxleaf) + align256(32 * cdivu(maxleaf, 128)) +
         align256(32 * (uint64_t)(n > 0 ? n : 1));
}

hipError_t hash_state(const brq_tensor_ref* t, int n, uint8_t* digest32, void* ws, hipStream_t s) {
  uint64_t maxleaf = 1;
  for (int i = 0; i < n; ++i) {
    uint64_t l = cdivu(tensor_bytes(t[i]), 4096);
    if (l > maxleaf) maxleaf = l;
  }
  uint8_t* bufA = (uint8_t*)ws;
  uint8_t* bufB = bufA + align256(32 * maxleaf);
  uint8_t* tdig = bufB + align256(32 * cdivu(maxleaf, 128));
  hipError_t e;
  for (int i = 0; i < n; ++i) {
    const uint64_t nb = tensor_bytes(t[i]);
    uint64_t cnt = nb == 0 ? 1 : cdivu(nb, 4096);
    hipLaunchKernelGGL(k_sha_leaves, dim3((unsigned)cdivu(cnt, 64)), dim3(64), 0, s,
                       (const uint8_t*)t[i].data, nb, cnt, bufA);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    uint8_t* cur = bufA;
    uint8_t* nxt = bufB;
    while (cnt > 1) {
      uint64_t nc = cdivu(cnt, 128);
      hipLaunchKernelGGL(k_sha_leaves, dim3((unsigned)cdivu(nc, 64)), dim3(64), 0, s, cur,
                         32 * cnt, nc, nxt);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      uint8_t* tmp = cur;
      cur = nxt;
      nxt = tmp;
      cnt = nc;
    }
    HeaderArg h{};
    int o = 0;
    h.bytes[o++] = 'B'; h.bytes[o++] = 'R'; h.bytes[o++] = 'Q'; h.bytes[o++] = '1';
    h.bytes[o++] = (uint8_t)t[i].dtype;
    h.bytes[o++] = (uint8_t)t[i].ndim;
    for (int d = 0; d < t[i].ndim; ++d)
      for (int b = 0; b < 8; ++b) h.bytes[o++] = (uint8_t)((uint64_t)t[i].dims[d] >> (8 * b));
    size_t nl = 0;
    while (t[i].name && t[i].name[nl]) ++nl;
    h.bytes[o++] = (uint8_t)(nl & 0xff);
    h.bytes[o++] = (uint8_t)(nl >> 8);
    for (size_t c = 0; c < nl; ++c) h.bytes[o++] = (uint8_t)t[i].name[c];
    h.len = o;
    hipLaunchKernelGGL(k_sha_header, dim3(1), dim3(1), 0, s, h, cur, tdig + 32 * i);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_sha_state, dim3(1), dim3(1), 0, s, tdig, n, digest32);
  return hipGetLastError();
}

}  // namespace brq
