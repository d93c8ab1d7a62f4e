// Device-side constants and helpers shared by the liboscar kernels (gfx950).
//
// Layout of one KV head's 5120-byte block in a page (documented in oscar.h):
//   [0, 2048) key codes, [2048, 4096) value codes (2 bits per code, 512 words
//   each), [4096, 5120) metadata: 16 bytes per token,
//   fp16 {sK0, loK0, sK1, loK1, sV0, loV0, sV1, loV1}.
// The key-code word order matches the i8 MFMA operand a wavefront lane needs
// (16 channels of one token per 32-bit word, one 128-bit load per lane covers
// four such words); the value-code word order holds 16 tokens of one channel
// per word for the f16 MFMA of the probability-value product.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "launch.h"

namespace oscar {

constexpr int D = 128;
constexpr int GROUP = 64;
constexpr int PAGE = 64;
constexpr int SINK = 64;
constexpr int WIN = 256;
constexpr int RING = 320;
static_assert(RING == 64 * RING_CHUNKS, "the ring is five 64-slot chunks");
constexpr int HEAD_BLOCK = 5120;
constexpr int KC_OFF = 0;
constexpr int VC_OFF = 2048;
constexpr int META_OFF = 4096;
constexpr int ROT_TERMS_OFF = D * D * 4;                 // 3 x bf16 [128][128] terms of R^T
constexpr int ROT_NMU_OFF = ROT_TERMS_OFF + 3 * D * D * 2;  // fp32 [128] -(mu . R), the key mean's shift
constexpr int ROT_HEAD_BYTES = ROT_NMU_OFF + D * 4;       // fp32 R [128][128] first

// ---------------------------------------------------------------- page layout

// Word index (0..511) of the key code (token j, channel c) in the key-code area.
__host__ __device__ inline int kc_word(int j, int c) {
  const int t = j >> 4, n = j & 15, g = c >> 6, kq = (c & 63) >> 4;
  return 256 * (t >> 1) + 4 * (16 * kq + n) + 2 * (t & 1) + g;
}
// Bit offset of channel c's key code inside its word.
__host__ __device__ inline int kc_bit(int c) {
  const int u = c & 15;
  return 8 * (u & 3) + 2 * (u >> 2);
}
// Word index of the value code (token j, channel c) in the value-code area.
__host__ __device__ inline int vc_word(int j, int c) {
  const int ct = c >> 4, n = c & 15, kq = (j & 31) >> 3;
  return 256 * (ct >> 2) + 4 * (16 * kq + n) + (ct & 3);
}
// Bit offset of token j's value code inside its word.
__host__ __device__ inline int vc_bit(int j) {
  const int s = j >> 5, kk = j & 7;
  return 2 * (4 * s + (kk >> 1)) + 16 * (kk & 1);
}

// ---------------------------------------------------------------- bf16

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// Round to nearest even; inputs are finite.
__device__ inline uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ---------------------------------------------------------------- quantizer
// Clip the group range [mn, mx] to width c*(mx-mn) about its midpoint and
// quantize to 4 levels with fp16 scale and minimum.  Each step is one IEEE
// fp32 operation rounded to nearest even, never fused, so the write path, the
// eviction path and any independent implementation of the same sequence agree
// bit for bit on identical inputs.
struct QParams {
  float lo;      // fp32 value of the stored fp16 minimum
  float inv;     // fp32(1 / s16), 0 when s16 == 0
  uint16_t s16;  // stored fp16 scale bits
  uint16_t lo16; // stored fp16 minimum bits
};

__device__ inline QParams quant_params(float mn, float mx, float c) {
#pragma clang fp contract(off)
  const float r = mx - mn;
  const float w = c * r;
  const float half = 0.5f * (r - w);
  const float lo32 = mn + half;
  const float s32 = w / 3.0f;
  const __half s16 = __float2half_rn(s32);
  const __half lo16 = __float2half_rn(lo32);
  QParams q;
  q.s16 = __half_as_ushort(s16);
  q.lo16 = __half_as_ushort(lo16);
  const float sf = __half2float(s16);
  q.lo = __half2float(lo16);
  q.inv = (sf != 0.0f) ? (1.0f / sf) : 0.0f;
  return q;
}

__device__ inline uint32_t quant_code(float x, const QParams& q) {
#pragma clang fp contract(off)
  const float t = (x - q.lo) * q.inv;
  const float r = __builtin_amdgcn_fmed3f(rintf(t), 0.0f, 3.0f);  // clamp to [0, 3]
  return static_cast<uint32_t>(r);
}

constexpr float C_K = 0.96f;
constexpr float C_V = 0.92f;

}  // namespace oscar
