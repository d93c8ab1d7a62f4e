// GPU twin of synth.bulk_keys / synth.bulk_values: seeded synthetic keys and
// values drawn in place on the device.  Input generation only; no part of the
// KV-cache method lives here.
//
// Definition (identical to the NumPy version in synth/__init__.py):
//   Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with key (key0, key1)
//   and counter (pair, pair >> 32, 0, 0), pair = token * 64 + channel / 2.
//   Even channels take output words 0,1, odd channels words 2,3; the draw is
//   z = (sum of the four 16-bit halves - 131070) * fp32(sqrt(3) / 65536).
//   Keys: bf16((z + mu[c]) * mult[c]); values: bf16(z); each step one fp32
//   operation rounded to nearest even, bf16 rounding to nearest even.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ inline void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t hi0 = __umulhi(M0, c[0]), lo0 = M0 * c[0];
    const uint32_t hi1 = __umulhi(M1, c[2]), lo1 = M1 * c[2];
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += W0; k1 += W1;
  }
}

__device__ inline float ih4(uint32_t a, uint32_t b) {
  const int32_t s = static_cast<int32_t>((a & 0xFFFFu) + (a >> 16) + (b & 0xFFFFu) + (b >> 16)) - 131070;
  return __fmul_rn(static_cast<float>(s), 0x1.bb67aep-16f /* fp32(sqrt(3)/65536) */);
}

__device__ inline uint16_t to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// One thread per (token, kv head, channel pair).  Destination layout [n_tokens][hkv][128].
__global__ void k_bulk_kv(uint16_t* __restrict__ k, uint16_t* __restrict__ v, int64_t n_tokens, int64_t token0,
                          int hkv, const uint32_t* __restrict__ key_k, const uint32_t* __restrict__ key_v,
                          uint32_t key1, const float* __restrict__ mu, const float* __restrict__ mult) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = n_tokens * hkv * 64;
  if (i >= total) return;
  const int cp = static_cast<int>(i & 63);
  const int64_t th = i >> 6;
  const int h = static_cast<int>(th % hkv);
  const int64_t t = th / hkv;
  const uint64_t pair = static_cast<uint64_t>(token0 + t) * 64u + static_cast<uint64_t>(cp);
  const size_t dst = (static_cast<size_t>(t) * hkv + h) * 128 + 2 * cp;
  if (k) {
    uint32_t c[4] = {static_cast<uint32_t>(pair), static_cast<uint32_t>(pair >> 32), 0u, 0u};
    philox10(c, key_k[h], key1);
    const float z0 = ih4(c[0], c[1]), z1 = ih4(c[2], c[3]);
    const int ch0 = 2 * cp, ch1 = 2 * cp + 1;
    const float x0 = __fmul_rn(__fadd_rn(z0, mu[h * 128 + ch0]), mult[h * 128 + ch0]);
    const float x1 = __fmul_rn(__fadd_rn(z1, mu[h * 128 + ch1]), mult[h * 128 + ch1]);
    k[dst] = to_bf16(x0);
    k[dst + 1] = to_bf16(x1);
  }
  if (v) {
    uint32_t c[4] = {static_cast<uint32_t>(pair), static_cast<uint32_t>(pair >> 32), 0u, 0u};
    philox10(c, key_v[h], key1);
    v[dst] = to_bf16(ih4(c[0], c[1]));
    v[dst + 1] = to_bf16(ih4(c[2], c[3]));
  }
}

}  // namespace

extern "C" int synth_bulk_kv(void* k, void* v, int64_t n_tokens, int64_t token0, int32_t hkv,
                             const void* key_k, const void* key_v, uint32_t key1, const void* mu,
                             const void* mult, void* stream) {
  if (n_tokens <= 0 || hkv <= 0) return -1;
  const int64_t total = n_tokens * hkv * 64;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return -1;
  hipLaunchKernelGGL(k_bulk_kv, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<uint16_t*>(k), static_cast<uint16_t*>(v),
                     n_tokens, token0, hkv, static_cast<const uint32_t*>(key_k), static_cast<const uint32_t*>(key_v),
                     key1, static_cast<const float*>(mu), static_cast<const float*>(mult));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
