// Write path: key rotation, clipping, per-token asymmetric INT2 quantization and
// page packing; BF16 sink/window stores; window eviction into INT2.
//
// Method: axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy
// barrier", section "어텐션 통계 기반 회전과 Triton 커널의 결합" - every new key
// is rotated by R_K, clipped with c_K = 0.96 (values c_V = 0.92), quantized per
// token to asymmetric INT2 in 64-channel groups; recent tokens stay BF16
// (section "Together AI, INT2 KV 캐시 시스템 'OSCAR' 공개").
#include "common.h"

namespace oscar {

// ------------------------------------------------------------------ utilities

__global__ void k_fill_i32(int32_t* dst, int64_t n, int32_t value) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = value;
}

__global__ void k_scatter(ScatterArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) a.dst[a.idx[i]] = a.val[i];
}

hipError_t launch_fill_i32(int32_t* dst, int64_t n, int32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_scatter, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ packing helpers

// Pack a 64-token head block from per-token codes (LDS bytes, one per code) and
// metadata halves.  256 threads; every word of the block is written, so slots
// without a token (codes 0, metadata 0) come out zero.
__device__ inline void pack_block(uint32_t* blk, const uint8_t (*kc)[D], const uint8_t (*vc)[D],
                                  const uint16_t (*meta)[8], int tid) {
  for (int w = tid; w < 512; w += 256) {
    // key word w: inverse of kc_word
    const int t2 = w >> 8, lane = (w & 255) >> 2, d = w & 3;
    const int t = 2 * t2 + (d >> 1), g = d & 1, kq = lane >> 4, n = lane & 15;
    const int j = 16 * t + n;
    uint32_t word = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = 64 * g + 16 * kq + u;
      word |= static_cast<uint32_t>(kc[j][c]) << kc_bit(c);
    }
    blk[(KC_OFF >> 2) + w] = word;
  }
  for (int w = tid; w < 512; w += 256) {
    // value word w: inverse of vc_word
    const int ct = 4 * (w >> 8) + (w & 3), lane = (w & 255) >> 2;
    const int kq = lane >> 4, n = lane & 15, c = 16 * ct + n;
    uint32_t word = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int j = 32 * s + 8 * kq + kk;
        word |= static_cast<uint32_t>(vc[j][c]) << vc_bit(j);
      }
    blk[(VC_OFF >> 2) + w] = word;
  }
  {
    const int w = tid;  // 256 metadata words: token w/4, halves 2*(w%4), 2*(w%4)+1
    const int j = w >> 2, h = 2 * (w & 3);
    blk[(META_OFF >> 2) + w] = static_cast<uint32_t>(meta[j][h]) | (static_cast<uint32_t>(meta[j][h + 1]) << 16);
  }
}

// ------------------------------------------------------------------ write kernel
// Grid (tiles of 64 positions, KV heads, sequences of this chunk); 256 threads.
// Tile i covers positions len0 + 64 i ... of its sequence.  For a sequence that
// was empty, tile i >= 1 holds INT2 indices 64 (i-1) ... = page i-1.

__global__ __launch_bounds__(256) void k_write(WriteArgs a) {
  const int tile = blockIdx.x, kvh = blockIdx.y, sl = blockIdx.z;
  const int tid = threadIdx.x;
  const WriteSeq sq = a.seqs[sl];
  const int n_here = min(PAGE, a.n_new - tile * PAGE);
  if (n_here <= 0) return;
  const int p0 = sq.len0 + tile * PAGE;
  const int len = sq.len0 + a.n_new;
  const int n_int2 = (sq.len0 == 0) ? max(0, len - RING) : 0;  // INT2 tokens of this call

  // kin (rotation input) and the code arrays (quantizer output) are never live together
  __shared__ union {
    uint16_t kin[PAGE][D];                 // bf16 keys of the tile
    struct {
      uint8_t kc[PAGE][D];
      uint8_t vc[PAGE][D];
    } q;
  } sm;
  __shared__ float x[PAGE][D + 1];         // rotated keys, fp32
  __shared__ uint16_t meta[PAGE][8];
  uint16_t (*kin)[D] = sm.kin;
  uint8_t (*kc)[D] = sm.q.kc;
  uint8_t (*vc)[D] = sm.q.vc;

  const size_t row = static_cast<size_t>(a.hkv) * D;
  const uint16_t* ksrc = a.k + (static_cast<size_t>(sq.src) * a.n_new + static_cast<size_t>(tile) * PAGE) * row + kvh * D;
  const uint16_t* vsrc = a.v + (static_cast<size_t>(sq.src) * a.n_new + static_cast<size_t>(tile) * PAGE) * row + kvh * D;
  for (int i = tid; i < PAGE * D; i += 256) {
    const int j = i / D, c = i % D;
    kin[j][c] = (j < n_here) ? ksrc[static_cast<size_t>(j) * row + c] : 0;
  }
  __syncthreads();

  // rotation x = k . R (fp32, VALU): thread owns channel c for 32 tokens
  {
    const float* rot = reinterpret_cast<const float*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES);
    const int c = tid & (D - 1), jh = tid >> 7;
    float acc[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) acc[t] = 0.0f;
    for (int i = 0; i < D; ++i) {
      const float r = rot[i * D + c];
#pragma unroll
      for (int t = 0; t < 32; ++t) acc[t] = fmaf(bf16_to_f32(kin[2 * t + jh][i]), r, acc[t]);
    }
#pragma unroll
    for (int t = 0; t < 32; ++t) x[2 * t + jh][c] = acc[t];
  }
  __syncthreads();

  // BF16 destinations: sink / window
  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  for (int i = tid; i < n_here * D; i += 256) {
    const int j = i / D, c = i % D, p = p0 + j;
    const bool int2 = (p >= SINK) && (p < SINK + n_int2);
    if (int2) continue;
    const int slot = (p < SINK) ? p : SINK + (p - SINK) % WIN;
    a.ring[ring_head + static_cast<size_t>(slot) * D + c] = f32_to_bf16(x[j][c]);
    a.ring[ring_head + static_cast<size_t>(RING + slot) * D + c] = vsrc[static_cast<size_t>(j) * row + c];
  }

  // INT2 destination: tokens j with SINK <= p0 + j < SINK + n_int2 (tile >= 1 of an empty sequence)
  int n_q = 0;
  if (n_int2 > 0 && p0 >= SINK) n_q = max(0, min(n_here, SINK + n_int2 - p0));
  if (n_q == 0) return;  // uniform across the block

  {
    // one (token, group, K/V) task per thread
    const int j = tid & 63, g = (tid >> 6) & 1, isv = tid >> 7;
    float mn = 0.0f, mx = 0.0f;
    float vals[GROUP];
    if (j < n_q) {
#pragma unroll
      for (int u = 0; u < GROUP; ++u)
        vals[u] = isv ? bf16_to_f32(vsrc[static_cast<size_t>(j) * row + 64 * g + u]) : x[j][64 * g + u];
      mn = vals[0];
      mx = vals[0];
#pragma unroll
      for (int u = 1; u < GROUP; ++u) {
        mn = fminf(mn, vals[u]);
        mx = fmaxf(mx, vals[u]);
      }
      const QParams q = quant_params(mn, mx, isv ? C_V : C_K);
      uint8_t (*dst)[D] = isv ? vc : kc;
#pragma unroll
      for (int u = 0; u < GROUP; ++u) dst[j][64 * g + u] = (q.s16 != 0) ? static_cast<uint8_t>(quant_code(vals[u], q)) : 0;
      meta[j][4 * isv + 2 * g] = q.s16;
      meta[j][4 * isv + 2 * g + 1] = q.lo16;
    } else {
      uint8_t (*dst)[D] = isv ? vc : kc;
      for (int u = 0; u < GROUP; ++u) dst[j][64 * g + u] = 0;
      meta[j][4 * isv + 2 * g] = 0;
      meta[j][4 * isv + 2 * g + 1] = 0;
    }
  }
  __syncthreads();
  const int page = a.page_table[static_cast<size_t>(sq.seq) * a.max_pages + (tile - 1)];
  uint32_t* blk = reinterpret_cast<uint32_t*>(a.pool + (static_cast<size_t>(page) * a.hkv + kvh) * HEAD_BLOCK);
  pack_block(blk, kc, vc, meta, tid);
}

hipError_t launch_write(const WriteArgs& a, int n_tiles, hipStream_t s) {
  hipLaunchKernelGGL(k_write, dim3(n_tiles, a.hkv, a.n_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ append (no INT2 output)
// Writes that only reach the BF16 sink / window (every append into a non-empty sequence, and a
// first write of at most 320 tokens).  Grid (KV heads, sequences of the chunk), 128 threads:
// thread c owns output channel c of every token; the rotation uses the same fp32 FMA order as
// the tile kernel above, so both paths store identical bf16 keys.

__global__ __launch_bounds__(128) void k_append(WriteArgs a) {
  const int kvh = blockIdx.x, sl = blockIdx.y, c = threadIdx.x;
  const WriteSeq sq = a.seqs[sl];
  __shared__ float kin[D];
  const float* rot = reinterpret_cast<const float*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES);
  const size_t row = static_cast<size_t>(a.hkv) * D;
  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  float rc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) rc[i] = rot[i * D + c];   // column c of R, kept in registers
  for (int t = 0; t < a.n_new; ++t) {
    const size_t src = (static_cast<size_t>(sq.src) * a.n_new + t) * row + kvh * D;
    __syncthreads();
    kin[c] = bf16_to_f32(a.k[src + c]);
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) acc = fmaf(kin[i], rc[i], acc);
    const int p = sq.len0 + t;
    const int slot = (p < SINK) ? p : SINK + (p - SINK) % WIN;
    a.ring[ring_head + static_cast<size_t>(slot) * D + c] = f32_to_bf16(acc);
    a.ring[ring_head + static_cast<size_t>(RING + slot) * D + c] = a.v[src + c];
  }
}

hipError_t launch_append(const WriteArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_append, dim3(a.hkv, a.n_seqs), dim3(128), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ eviction
// Grid (KV heads, sequences); 256 threads.  Tokens are evicted one after the
// other: INT2 index i takes ring slot 64 + i % 256 (the oldest window token).

__global__ __launch_bounds__(256) void k_evict(EvictArgs a) {
  const int kvh = blockIdx.x, sl = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const EvictSeq sq = a.seqs[sl];
  __shared__ uint8_t codes[2][D];
  __shared__ uint16_t meta[8];
  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  for (int e = 0; e < a.n_evict; ++e) {
    const int i = sq.n_int2 + e;
    const int slot = i & (PAGE - 1);
    const int page = a.page_table[static_cast<size_t>(sq.seq) * a.max_pages + i / PAGE];
    uint32_t* blk = reinterpret_cast<uint32_t*>(a.pool + (static_cast<size_t>(page) * a.hkv + kvh) * HEAD_BLOCK);
    if (slot == 0) {
      for (int w = tid; w < HEAD_BLOCK / 4; w += 256) blk[w] = 0;
      __threadfence_block();
    }
    __syncthreads();
    const int rs = SINK + (i % WIN);
    // wave wv: task (isv = wv >> 1, group = wv & 1); lane holds one channel
    const int isv = wv >> 1, g = wv & 1, c = 64 * g + lane;
    const float xv = bf16_to_f32(a.ring[ring_head + (static_cast<size_t>(isv) * RING + rs) * D + c]);
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
      // value word of channel cc: read-modify-write of this token's 2 bits
      const int cc = tid - 8;
      uint32_t* wp = blk + (VC_OFF >> 2) + vc_word(slot, cc);
      const int b = vc_bit(slot);
      *wp = (*wp & ~(3u << b)) | (static_cast<uint32_t>(codes[1][cc]) << b);
    } else if (tid < 8 + D + 4) {
      const int m = tid - 8 - D;
      blk[(META_OFF >> 2) + 4 * slot + m] = static_cast<uint32_t>(meta[2 * m]) | (static_cast<uint32_t>(meta[2 * m + 1]) << 16);
    }
    __threadfence_block();
    __syncthreads();
  }
}

hipError_t launch_evict(const EvictArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_evict, dim3(a.hkv, a.n_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
