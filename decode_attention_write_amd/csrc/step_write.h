// Device routines of the decode step's write, shared by the write kernels and the fused
// decode-step kernel (write + query preparation in one launch).
//
// Method: axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy barrier", section
// "어텐션 통계 기반 회전과 Triton 커널의 결합" (every new key rotated by R_K, clipped and
// quantized to INT2); recent tokens stay BF16 and the oldest window token moves to INT2
// (techllm, "KV cache compression", section "OSCAR").
#pragma once

#include "common.h"

namespace oscar {

// ------------------------------------------------------------------ single-token key rotation
// Output channel c of one key's rotation, shift_c + sum_i k_i R_ic, with column c of R in
// registers: four interleaved partial sums (i mod 4) added at the end, so the 128 fused
// multiply-adds form four independent chains instead of one.
__device__ inline float rotate_channel(const float* kin, const float* rc, float shift) {
  float p[4] = {shift, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < D; ++i) p[i & 3] = fmaf(kin[i], rc[i], p[i & 3]);
  return (p[0] + p[1]) + (p[2] + p[3]);
}

// ------------------------------------------------------------------ eviction
// One token of one (sequence, KV head) moves from the window to INT2: INT2 index i takes ring
// slot 64 + i % 256 (the oldest window token).  256 threads: thread t holds channel t % 128 of
// the key (t < 128) or the value (t >= 128).

// This thread's ring element of the token that INT2 index i evicts.
__device__ inline float evict_value(const uint16_t* ring, int hkv, int seq, int kvh, int i) {
  const int tid = threadIdx.x, isv = tid >> 7, c = tid & (D - 1);
  const size_t ring_head = (static_cast<size_t>(seq) * hkv + kvh) * 2 * RING * D;
  return bf16_to_f32(ring[ring_head + (static_cast<size_t>(isv) * RING + SINK + (i % WIN)) * D + c]);
}

// Quantizes and stores the evicted token (xv: this thread's ring element, from evict_value) into
// slot i % 64 of `page`.  A page's slot 0 clears the whole block first (pages are recycled);
// later slots only add their bits: the key words and metadata of a token are whole words, the
// value words hold 16 tokens each and take the token's codes by an atomic OR, so no word is read
// back.  Uses LDS scratch codes/meta; ends with a barrier.
__device__ inline void evict_one(uint8_t* pool, int hkv, int page, int kvh, int i, float xv, uint8_t (*codes)[D],
                                 uint16_t* meta) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int slot = i & (PAGE - 1);
  uint32_t* blk = reinterpret_cast<uint32_t*>(pool + (static_cast<size_t>(page) * hkv + kvh) * HEAD_BLOCK);
  if (slot == 0) {
    for (int w = tid; w < HEAD_BLOCK / 4; w += 256) blk[w] = 0;
    __threadfence_block();
  }
  __syncthreads();
  // wave wv: task (isv = wv >> 1, group = wv & 1); lane holds one channel
  const int isv = wv >> 1, g = wv & 1, c = 64 * g + lane;
  float mn = xv, mx = xv;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, 64));
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  const QParams q = quant_params(mn, mx, isv ? C_V : C_K);
  codes[isv][c] = (q.s16 != 0) ? static_cast<uint8_t>(quant_code(xv, q)) : 0;
  if (lane == 0) {
    meta[4 * isv + 2 * g] = q.s16;
    meta[4 * isv + 2 * g + 1] = q.lo16;
  }
  __syncthreads();
  if (tid < 8) {
    // key words of this token: (g, kq) -> word kc_word(slot, 64 g + 16 kq)
    const int gg = tid >> 2, kq = tid & 3;
    uint32_t word = 0;
    for (int u = 0; u < 16; ++u) {
      const int cc = 64 * gg + 16 * kq + u;
      word |= static_cast<uint32_t>(codes[0][cc]) << kc_bit(cc);
    }
    blk[(KC_OFF >> 2) + kc_word(slot, 64 * gg + 16 * kq)] = word;
  } else if (tid < 8 + D) {
    // value word of channel cc: this token's 2 bits, whose place is still zero
    const int cc = tid - 8;
    const uint32_t bits = static_cast<uint32_t>(codes[1][cc]) << vc_bit(slot);
    if (bits != 0)
      __hip_atomic_fetch_or(blk + (VC_OFF >> 2) + vc_word(slot, cc), bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (tid < 8 + D + 4) {
    const int m = tid - 8 - D;
    blk[(META_OFF >> 2) + 4 * slot + m] = static_cast<uint32_t>(meta[2 * m]) | (static_cast<uint32_t>(meta[2 * m + 1]) << 16);
  }
  __threadfence_block();
  __syncthreads();
}

// ------------------------------------------------------------------ decode-step write
// One (KV head, sequence of the chunk) per 256-thread work-group: the eviction of k_evict (when
// the window is full) and the single-token append of k_append.  Every load is issued first
// (the evicted token's ring element, and for thread c < 128 the new token's key and value and
// column c of R_K), so the step waits for memory once; the evicted token's page comes with the
// plan.  The new token lands in the ring slot the eviction has just read (window position
// 64 + n_int2 + 256 maps to slot 64 + n_int2 % 256), so it is written only after the eviction's
// barriers.
__device__ inline void step_write_block(const StepArgs& a, int kvh, int sl) {
  const int tid = threadIdx.x;
  const StepSeq sq = a.seqs[sl];
  __shared__ uint8_t codes[2][D];
  __shared__ uint16_t meta[8];
  __shared__ float kin[D];
  const size_t src = (static_cast<size_t>(sq.src) * a.hkv + kvh) * D;
  float rc[D];
  float shift = 0.0f;
  uint16_t vraw = 0;
  if (tid < D) {
    const float* rot = reinterpret_cast<const float*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES);
#pragma unroll
    for (int i = 0; i < D; ++i) rc[i] = rot[i * D + tid];   // column tid of R
    shift = rot[ROT_NMU_OFF / 4 + tid];                       // -(mu . R)_tid, the key mean's shift
    kin[tid] = bf16_to_f32(a.k[src + tid]);
    vraw = a.v[src + tid];
  }
  const float xv = sq.evict ? evict_value(a.ring, a.hkv, sq.seq, kvh, sq.n_int2) : 0.0f;
  if (sq.evict) evict_one(a.pool, a.hkv, sq.page, kvh, sq.n_int2, xv, codes, meta);
  __syncthreads();
  if (tid < D) {
    const float acc = rotate_channel(kin, rc, shift);
    const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
    const int p = sq.len0;
    const int slot = (p < SINK) ? p : SINK + (p - SINK) % WIN;
    a.ring[ring_head + static_cast<size_t>(slot) * D + tid] = f32_to_bf16(acc);
    a.ring[ring_head + static_cast<size_t>(RING + slot) * D + tid] = vraw;
  }
}

}  // namespace oscar
