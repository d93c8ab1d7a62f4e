// Write path: key rotation, clipping, per-token asymmetric INT2 quantization and
// page packing; BF16 sink/window stores; window eviction into INT2.
//
// Method: axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy
// barrier", section "어텐션 통계 기반 회전과 Triton 커널의 결합" - every new key
// is rotated by R_K, clipped with c_K = 0.96 (values c_V = 0.92), quantized per
// token to asymmetric INT2 in 64-channel groups; recent tokens stay BF16
// (section "Together AI, INT2 KV 캐시 시스템 'OSCAR' 공개").
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "oscar.h"
#include "step_write.h"

namespace oscar {

static_assert(ROT_HEAD_BYTES == OSCAR_ROT_HEAD_BYTES, "rotation block layout");

// ------------------------------------------------------------------ utilities

__global__ void k_fill_i32(int32_t* dst, int64_t n, int32_t value) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = value;
}

__global__ void k_scatter(ScatterArgs a) {
  const int i = threadIdx.x;
  if (i < a.n) a.dst[a.idx[i]] = a.val[i];
}

__global__ void k_run(RunArgs a) {
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) a.dst[i] = a.val[i];
}

hipError_t launch_fill_i32(int32_t* dst, int64_t n, int32_t value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_fill_i32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

hipError_t launch_run(const RunArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_run, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_scatter, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ write kernel
// Grid (groups of tiles_per_wg tiles of 64 positions, KV heads, sequences of this chunk); 512
// threads in 8 waves.  Tile i covers positions len0 + 64 i ... of its sequence.  For a sequence
// that was empty, tile i >= 1 holds INT2 indices 64 (i-1) ... = page i-1.  launch_write sizes the
// groups so that all work-groups are resident at once (one residency round).
//
// Rotation on the matrix cores, transposed: x^T = R^T k^T with v_mfma_f32_16x16x32_bf16.  The A
// operand is R^T as three bf16 terms r0 = bf16(R^T), r1 = bf16(R^T - r0), r2 = bf16(R^T - r0 - r1),
// so |R^T - r0 - r1 - r2| <= 2^-24 |R^T|; the B operand is the bf16 key tile as it is.  The
// products are exact in fp32 and accumulate in fp32 (12 instructions of 32 products each, the
// small terms first), starting from -(mu . R) when a key mean mu is set (zero otherwise).  Wave w
// owns output channels 16 w .. 16 w + 15 of all 64 tokens and keeps its A operand in registers for
// all tiles of the work-group; lane (q4, n16) holds channels 16 w + 4 q4 + e (e = 0..3) of the
// tokens 16 nt + n16 (nt = 0..3), and reads the values of the same positions from the value tile.
//
// Quantization works in that register layout.  Range per (token, 64-channel group): each lane
// reduces its 4 channels, the 4 rows of a wave are combined by lane swaps (v_permlane32_swap,
// v_permlane16_swap), the 4 waves of a group through LDS; one thread per (token, group, K or V)
// derives the fp16 scale and minimum, stores the metadata word and publishes (minimum, 1/scale).
// Code of x: z = (x - lo) * (1/s) + 2^23 holds the level rounded to the nearest integer in its low
// bits (the sum's unit in the last place is 1); clamped to 2^23 + [0, 3], z's bit pattern shifted
// to the code's place is summed over the lanes that share a 32-bit word.  The fields are disjoint, so
// the sum equals the bitwise or of the codes plus the shifted 2^23 patterns, a constant that is
// taken off at the end.  A key word (16 channels of one token) spans the 4 rows of a wave; a
// value word (16 tokens of one channel) spans the 8 lanes of a half-row.

constexpr int KS = D + 8;              // 16-bit row stride of the key / value tiles
constexpr float Z0F = 8388608.0f;      // 2^23
constexpr uint32_t Z0 = 0x4B000000u;   // its bit pattern

// The shifted 2^23 patterns a finished word carries (mod 2^32): key words hold (row q4, channel e)
// at bit 8 e + 2 q4; value words hold (lane kk of the half-row, token half s) at bit
// 8 s + 2 (kk >> 1) + 16 (kk & 1).
constexpr uint32_t key_word_bias() {
  uint32_t b = 0;
  for (int q = 0; q < 4; ++q)
    for (int e = 0; e < 4; ++e) b += Z0 << (8 * e + 2 * q);
  return b;
}
constexpr uint32_t value_word_bias() {
  uint32_t b = 0;
  for (int kk = 0; kk < 8; ++kk)
    for (int s = 0; s < 2; ++s) b += Z0 << (8 * s + 2 * (kk >> 1) + 16 * (kk & 1));
  return b;
}

typedef __bf16 v8bf_w __attribute__((ext_vector_type(8)));
typedef float v4f_w __attribute__((ext_vector_type(4)));
typedef float v2f_w __attribute__((ext_vector_type(2)));
typedef unsigned int v4u_w __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_w __attribute__((ext_vector_type(2)));
typedef int v4i_w __attribute__((ext_vector_type(4)));

// A copy of a lane value the compiler cannot see through: indices derived from it are formed where
// they are used instead of being kept live across the tile loop (which spilled).
__device__ inline int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// 2^23 + code of x under (lo, inv), as a bit pattern.  t = (x - lo) * inv in two fp32 roundings,
// as the eviction path's quant_code takes it (an exact tie k + 1/2 of (x - lo) / s stays a tie in
// fp32 and goes to even on both paths; a fused multiply-add would break it by the error of inv);
// t + 2^23 then rounds t to the nearest integer, ties to even, like rintf.  CLAMP false skips the
// clamp to [0, 3] where the caller knows every level of the group already lies in it.
template <bool CLAMP>
__device__ inline uint32_t code_bits(float x, float lo, float inv) {
#pragma clang fp contract(off)
  const float z = (x - lo) * inv + Z0F;
  return __float_as_uint(CLAMP ? __builtin_amdgcn_fmed3f(z, Z0F, Z0F + 3.0f) : z);
}

// fp32 minimum / maximum as single instructions: with fminf / fmaxf the compiler first quiets
// possible signalling NaNs of every operand (one more instruction each); the inputs here are finite.
__device__ inline float vmin(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float vmin3(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// op(x, y) over rows r and r ^ 2 (lanes l, l ^ 32) of two registers at once: rows 0-1 of the
// result hold x's, rows 2-3 y's
__device__ inline float fmin32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return vmin(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float fmax32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// op over rows r and r ^ 1: rows 0 and 2 of the result hold x's, rows 1 and 3 y's
__device__ inline float fmin16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return vmin(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float fmax16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline uint32_t add32(uint32_t x, uint32_t y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  return r[0] + r[1];
}
__device__ inline uint32_t add16(uint32_t x, uint32_t y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  return r[0] + r[1];
}
// Transposing sum of a pair over lane pairs (l, partner(l)): lanes with sel hold a's sum, the
// others b's (partner(l) has the opposite sel)
template <int CTRL>
__device__ inline uint32_t pair_sum(uint32_t a, uint32_t b, bool sel) {
  const uint32_t keep = sel ? b : a, give = sel ? a : b;
  return keep + static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(give), CTRL, 0xF, 0xF, false));
}

// Codes of one tile for this lane's positions (acc: rotated keys, vv: values, both [token column
// nt][channel e]) packed into one key word and one value word, stored to the page block.
template <bool CLAMP>
__device__ inline void write_codes(uint32_t* blk, const v4f_w* acc, const v4f_w* vv, const v2f_w (*prm)[PAGE][2],
                                   int lane_in, int grp, int kq) {
  const int lane = opaque(lane_in), q4 = lane >> 4, n16 = lane & 15;
  // key words: the 4 codes of token 16 nt + n16 at bits 8 e + 2 q4, summed over the 4 rows
  uint32_t kw[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const v2f_w pk = prm[0][16 * nt + n16][grp];
    const v4f_w x = acc[nt];
    uint32_t w = code_bits<CLAMP>(x.x, pk.x, pk.y);
    w += code_bits<CLAMP>(x.y, pk.x, pk.y) << 8;
    w += code_bits<CLAMP>(x.z, pk.x, pk.y) << 16;
    w += code_bits<CLAMP>(x.w, pk.x, pk.y) << 24;
    kw[nt] = w << (2 * q4);
  }
  const uint32_t kword = add16(add32(kw[0], kw[1]), add32(kw[2], kw[3])) - key_word_bias();
  {
    // this lane's word after the swaps: token 16 t + n16 with t = [0, 2, 1, 3][row]
    const int t = ((q4 & 1) << 1) | (q4 >> 1);
    blk[(KC_OFF >> 2) + 256 * (t >> 1) + 4 * (16 * kq + n16) + 2 * (t & 1) + grp] = kword;
  }
  // value words: code of (token 16 nt + n16, channel e) at bit 8 (nt >> 1) + vsh of the partial
  // word (e, nt & 1), summed over the 8 lanes of the half-row
  const int kk = lane & 7;
  const int vsh = 2 * (kk >> 1) + 16 * (kk & 1);  // bit of token 16 nt + n16, nt < 2
  uint32_t pv[8];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const v2f_w pq = prm[1][16 * nt + n16][grp];
    const float v[4] = {vv[nt].x, vv[nt].y, vv[nt].z, vv[nt].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t c = code_bits<CLAMP>(v[e], pq.x, pq.y);
      if (nt < 2)
        pv[2 * e + nt] = c << vsh;
      else
        pv[2 * e + (nt & 1)] += c << (vsh + 8);
    }
  }
  // the 8 partial words (e, h) of the 8 lanes of a half-row -> one finished word per lane: level
  // 1 keeps h = sel0, level 2 e & 1 = sel1, level 3 e >> 1 = sel2; the selections of the upper
  // quad are inverted so that half-row mirror partners hold the same word
  const bool sel0 = ((lane ^ (lane >> 2)) & 1) != 0;
  const bool sel1 = (((lane >> 1) ^ (lane >> 2)) & 1) != 0;
  const bool sel2 = ((lane >> 2) & 1) != 0;
  uint32_t q[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) q[m] = pair_sum<0xB1>(pv[2 * m], pv[2 * m + 1], sel0);  // lanes l, l ^ 1
  const uint32_t r0 = pair_sum<0x4E>(q[0], q[1], sel1);                                // lanes l, l ^ 2
  const uint32_t r1 = pair_sum<0x4E>(q[2], q[3], sel1);
  const uint32_t vword = pair_sum<0x141>(r0, r1, sel2) - value_word_bias();             // lanes l, 7 - l
  // word of channel 16 w + 4 q4 + e, e = 2 sel2 + sel1, token quarter 2 sel0 + (n16 >> 3)
  const int e = 2 * static_cast<int>(sel2) + static_cast<int>(sel1);
  const int vq = 2 * static_cast<int>(sel0) + ((lane >> 3) & 1);
  blk[(VC_OFF >> 2) + 256 * grp + 4 * (16 * vq + 4 * q4 + e) + kq] = vword;
}

__global__ __launch_bounds__(512, 4) void k_write(WriteArgs a) {
  const int kvh = blockIdx.y, sl = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q4 = lane >> 4, n16 = lane & 15;
  const WriteSeq sq = a.seqs[sl];
  const int n_tiles = (a.n_new + PAGE - 1) / PAGE;
  const int tile0 = blockIdx.x * a.tiles_per_wg;
  if (tile0 >= n_tiles) return;
  const int tile1 = min(tile0 + a.tiles_per_wg, n_tiles);
  const int len = sq.len0 + a.n_new;
  const int n_int2 = (sq.len0 == 0) ? max(0, len - RING) : 0;  // INT2 tokens of this call
  const int grp = wave >> 2, kq = wave & 3;  // this wave's 64-channel group and 16-channel quarter

  __shared__ uint16_t tk[PAGE][KS];        // bf16 keys of the tile
  __shared__ uint16_t tv[PAGE][KS];        // bf16 values of the tile
  __shared__ v2f_w part[2][4][2][PAGE];    // (min, max) per (K/V, wave of the group, group, token)
  __shared__ v2f_w prm[2][PAGE][2];        // (fp32 minimum, 1/scale) per (K/V, token, group)
  __shared__ int need_clamp[4];            // per parameter wave: some level may fall outside [0, 3]
  __shared__ float nmu[D];                 // -(mu . R): the key mean's shift, starts every accumulator

  // A operands: R^T rows 16 w + n16, 4 K-steps of 32 input channels, 3 terms
  const uint8_t* rblk = a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES;
  const uint16_t* terms = reinterpret_cast<const uint16_t*>(rblk + ROT_TERMS_OFF);
  if (tid < D) nmu[tid] = reinterpret_cast<const float*>(rblk + ROT_NMU_OFF)[tid];  // read after the first barrier
  v8bf_w aop[4][3];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int t = 0; t < 3; ++t)
      aop[ks][t] = *reinterpret_cast<const v8bf_w*>(terms + t * D * D + (16 * wave + n16) * D + 32 * ks + 8 * q4);

  const uint32_t row_bytes = static_cast<uint32_t>(a.hkv) * D * 2;
  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  // A 64 x 128 bf16 tile (keys or values) moves global -> registers (2 x 16 bytes per thread) ->
  // LDS.  Inputs are read once: they go with the non-temporal hint.  The INT2 words are stored as
  // plain 4-byte stores, which the L2 merges into whole lines (with the non-temporal hint they
  // reached memory as partial lines: 1.5 x the page bytes written, at the same speed).  When a tile's buffers have been read, the next tile goes from the
  // registers to LDS and the loads of the one after it are issued: in flight for a whole tile of
  // rotation and quantization.  Loads are never
  // conditional (rows past the call's tokens re-read the last row and are zeroed when stored; past
  // the work-group's last tile every lane reads the first row of its last tile, whose registers
  // are then never used: 512 bytes instead of a tile), which keeps the compiler's waits on them
  // counted ones.  The tile's base is uniform; each lane adds a 32-bit byte offset.
  auto issue = [&](int t_req, v4u_w* kw, v4u_w* vw) {
    const int t = min(t_req, tile1 - 1);
    const int nh = (t_req >= tile1) ? 1 : min(PAGE, a.n_new - t * PAGE);
    const size_t base = ((static_cast<size_t>(sq.src) * a.n_new + static_cast<size_t>(t) * PAGE) * a.hkv + kvh) * D * 2;
    const char* kb = reinterpret_cast<const char*>(a.k) + base;
    const char* vb = reinterpret_cast<const char*>(a.v) + base;
    const int t_ = opaque(tid);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = t_ + 512 * r;
      const uint32_t off = __umul24(static_cast<uint32_t>(min(i >> 4, nh - 1)), row_bytes) + 16u * static_cast<uint32_t>(i & 15);
      kw[r] = __builtin_nontemporal_load(reinterpret_cast<const v4u_w*>(kb + off));
      vw[r] = __builtin_nontemporal_load(reinterpret_cast<const v4u_w*>(vb + off));
    }
  };
  // registers -> LDS; rows past the call's tokens zeroed (LDS stores only)
  auto stash = [&](int t, const v4u_w* kw, const v4u_w* vw) {
    const int nh = min(PAGE, a.n_new - t * PAGE);
    const int t_ = opaque(tid);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = t_ + 512 * r, j = i >> 4, c8 = 8 * (i & 15);
      *reinterpret_cast<v4u_w*>(&tk[j][c8]) = kw[r];
      *reinterpret_cast<v4u_w*>(&tv[j][c8]) = vw[r];
    }
    if (nh < PAGE) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = t_ + 512 * r, j = i >> 4, c8 = 8 * (i & 15);
        if (j >= nh) {
          const int z_ = opaque(0);
          *reinterpret_cast<v4u_w*>(&tk[j][c8]) = v4u_w{0u, 0u, 0u, 0u} + static_cast<uint32_t>(z_);
          *reinterpret_cast<v4u_w*>(&tv[j][c8]) = v4u_w{0u, 0u, 0u, 0u} + static_cast<uint32_t>(z_);
        }
      }
    }
  };
  // page ids through the scalar cache (the table is not written by this kernel)
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + static_cast<size_t>(sq.seq) * a.max_pages);

  v4u_w kreg[2], vreg[2];
  issue(tile0, kreg, vreg);
  stash(tile0, kreg, vreg);
  issue(tile0 + 1, kreg, vreg);
  for (int tile = tile0; tile < tile1; ++tile) {
    const int n_here = min(PAGE, a.n_new - tile * PAGE);
    const int p0 = sq.len0 + tile * PAGE;
    // INT2 destination: tokens j with SINK <= p0 + j < SINK + n_int2 (tile >= 1 of an empty
    // sequence).  Only such a tile reads a page id, so the reads stay within the row's first
    // ceil(n_int2 / 64) entries.
    int n_q = 0;
    if (n_int2 > 0 && p0 >= SINK) n_q = max(0, min(n_here, SINK + n_int2 - p0));
    const int page = (n_q > 0) ? ptab[tile - 1] : 0;
    __syncthreads();  // the tile is in LDS

    // rotation: 4 token columns of 16, each accumulator starting from the key mean's shift; values
    // of the same positions
    v4f_w acc[4];
    v2u_w vp[4];
    const v4f_w shift = *reinterpret_cast<const v4f_w*>(&nmu[16 * wave + 4 * q4]);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      v8bf_w b[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) b[ks] = *reinterpret_cast<const v8bf_w*>(&tk[16 * nt + n16][32 * ks + 8 * q4]);
      acc[nt] = shift;
#pragma unroll
      for (int t = 2; t >= 0; --t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[ks][t], b[ks], acc[nt], 0, 0, 0);
      vp[nt] = *reinterpret_cast<const v2u_w*>(&tv[16 * nt + n16][16 * wave + 4 * q4]);
    }

    // BF16 destinations: sink / window (tiles holding such positions only); 4 channels of one
    // token per lane and store
    const bool any_bf16 = (p0 < SINK) || (p0 + n_here > SINK + n_int2);
    if (any_bf16) {
      const int l_ = opaque(lane);
      const int ln16 = l_ & 15, lch = 16 * wave + 4 * (l_ >> 4);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = 16 * nt + ln16, p = p0 + j;
        const bool int2 = (p >= SINK) && (p < SINK + n_int2);
        if (j < n_here && !int2) {
          const int slot = (p < SINK) ? p : SINK + (p - SINK) % WIN;
          const v2u_w kw = {static_cast<uint32_t>(f32_to_bf16(acc[nt].x)) | (static_cast<uint32_t>(f32_to_bf16(acc[nt].y)) << 16),
                            static_cast<uint32_t>(f32_to_bf16(acc[nt].z)) | (static_cast<uint32_t>(f32_to_bf16(acc[nt].w)) << 16)};
          const v2u_w vw = vp[nt];
          *reinterpret_cast<v2u_w*>(a.ring + ring_head + static_cast<size_t>(slot) * D + lch) = kw;
          *reinterpret_cast<v2u_w*>(a.ring + ring_head + static_cast<size_t>(RING + slot) * D + lch) = vw;
        }
      }
    }

    if (n_q > 0) {  // uniform across the block
      // range of the lane's 4 channels per token, then over the wave's 4 rows: after the two
      // swap levels row r holds token column kt(r) = [0, 2, 1, 3][r]
      float kmn[4], kmx[4], vmn[4], vmx[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const v4f_w vvv = {__uint_as_float(vp[nt].x << 16), __uint_as_float(vp[nt].x & 0xFFFF0000u),
                           __uint_as_float(vp[nt].y << 16), __uint_as_float(vp[nt].y & 0xFFFF0000u)};
        kmn[nt] = vmin3(acc[nt].x, acc[nt].y, vmin(acc[nt].z, acc[nt].w));
        kmx[nt] = vmax3(acc[nt].x, acc[nt].y, vmax(acc[nt].z, acc[nt].w));
        vmn[nt] = vmin3(vvv.x, vvv.y, vmin(vvv.z, vvv.w));
        vmx[nt] = vmax3(vvv.x, vvv.y, vmax(vvv.z, vvv.w));
      }
      const float kmn_ = fmin16(fmin32(kmn[0], kmn[1]), fmin32(kmn[2], kmn[3]));
      const float kmx_ = fmax16(fmax32(kmx[0], kmx[1]), fmax32(kmx[2], kmx[3]));
      const float vmn_ = fmin16(fmin32(vmn[0], vmn[1]), fmin32(vmn[2], vmn[3]));
      const float vmx_ = fmax16(fmax32(vmx[0], vmx[1]), fmax32(vmx[2], vmx[3]));
      const int l_ = opaque(lane), r_ = l_ >> 4;
      const int tok = 16 * (((r_ & 1) << 1) | (r_ >> 1)) + (l_ & 15);
      part[0][kq][grp][tok] = v2f_w{kmn_, kmx_};
      part[1][kq][grp][tok] = v2f_w{vmn_, vmx_};
    }
    __syncthreads();  // ranges published; every read of the tile buffers is done

    // the next tile into LDS (loaded during the previous tile), then the loads of the one after
    stash(min(tile + 1, tile1 - 1), kreg, vreg);
    issue(tile + 2, kreg, vreg);

    if (n_q > 0) {
      uint32_t* blk = reinterpret_cast<uint32_t*>(a.pool + (static_cast<size_t>(page) * a.hkv + kvh) * HEAD_BLOCK);
      // quantizer parameters: thread t < 256 takes (token t >> 2, K/V (t >> 1) & 1, group t & 1),
      // which is also the order of the metadata words
      if (tid < 256) {
        const int t_ = opaque(tid);
        const int j = t_ >> 2, isv = (t_ >> 1) & 1, g = t_ & 1;
        float mn = vmin3(part[isv][0][g][j].x, part[isv][1][g][j].x, vmin(part[isv][2][g][j].x, part[isv][3][g][j].x));
        float mx = vmax3(part[isv][0][g][j].y, part[isv][1][g][j].y, vmax(part[isv][2][g][j].y, part[isv][3][g][j].y));
        float lo = 0.0f, inv = 0.0f;
        uint32_t mword = 0u;  // slots without a token: minimum 0, reciprocal scale 0 -> code 0
        if (j < n_q) {
          const QParams qp = quant_params(mn, mx, isv ? C_V : C_K);
          lo = qp.lo;
          inv = qp.inv;  // 0 when the stored scale is 0: every code is then 0
          mword = static_cast<uint32_t>(qp.s16) | (static_cast<uint32_t>(qp.lo16) << 16);
        }
        blk[(META_OFF >> 2) + t_] = mword;
        prm[isv][j][g] = v2f_w{lo, inv};
        // levels are monotone in x: if the group's smallest and largest values land in [0, 3]
        // unclamped, every value of the group does
        const bool in_range = (code_bits<false>(mn, lo, inv) >= Z0) && (code_bits<false>(mx, lo, inv) <= Z0 + 3u);
        const uint64_t ok = __ballot(in_range);
        if ((t_ & 63) == 0) need_clamp[t_ >> 6] = (ok != ~0ull) ? 1 : 0;
      }
      __syncthreads();  // parameters published

      const v4i_w nc = *reinterpret_cast<const v4i_w*>(need_clamp);
      v4f_w vv[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        vv[nt] = v4f_w{__uint_as_float(vp[nt].x << 16), __uint_as_float(vp[nt].x & 0xFFFF0000u),
                       __uint_as_float(vp[nt].y << 16), __uint_as_float(vp[nt].y & 0xFFFF0000u)};
      if ((nc.x | nc.y | nc.z | nc.w) != 0)
        write_codes<true>(blk, acc, vv, prm, lane, grp, kq);
      else
        write_codes<false>(blk, acc, vv, prm, lane, grp, kq);
    }
  }
}

// Work-groups of k_write that the device holds at once (occupancy query, cached per device).
static int write_resident_workgroups() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n_cu = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_write, 512, 0) != hipSuccess) return 0;
    cache[dev] = n_cu * per_cu;
  }
  return cache[dev];
}

hipError_t launch_write(const WriteArgs& a_in, int n_tiles, hipStream_t s) {
  WriteArgs a = a_in;
  const int64_t total = static_cast<int64_t>(n_tiles) * a.hkv * a.n_seqs;
  const int slots = write_resident_workgroups();
  a.tiles_per_wg = slots > 0 ? static_cast<int32_t>(std::max<int64_t>(1, (total + slots - 1) / slots)) : 8;
  const int groups = (n_tiles + a.tiles_per_wg - 1) / a.tiles_per_wg;
  hipLaunchKernelGGL(k_write, dim3(groups, a.hkv, a.n_seqs), dim3(512), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ append (no INT2 output)
// Writes that only reach the BF16 sink / window (every append into a non-empty sequence, and a
// first write of at most 320 tokens).  Grid (KV heads, sequences of the chunk), 128 threads:
// thread c owns output channel c of every token; fp32 VALU rotation (a single token per sequence
// and head is too little work for the matrix cores).

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
  const float shift = reinterpret_cast<const float*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES + ROT_NMU_OFF)[c];
  for (int t = 0; t < a.n_new; ++t) {
    const size_t src = (static_cast<size_t>(sq.src) * a.n_new + t) * row + kvh * D;
    __syncthreads();
    kin[c] = bf16_to_f32(a.k[src + c]);
    __syncthreads();
    const float acc = rotate_channel(kin, rc, shift);  // shift: -(mu . R)_c, +0 without a key mean
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
// Grid (KV heads, sequences); 256 threads.  Tokens are evicted one after the other.
__global__ __launch_bounds__(256) void k_evict(EvictArgs a) {
  const int kvh = blockIdx.x, sl = blockIdx.y;
  const EvictSeq sq = a.seqs[sl];
  __shared__ uint8_t codes[2][D];
  __shared__ uint16_t meta[8];
  const int32_t* ptab = a.page_table + static_cast<size_t>(sq.seq) * a.max_pages;
  for (int e = 0; e < a.n_evict; ++e) {
    const int i = sq.n_int2 + e;
    const float xv = evict_value(a.ring, a.hkv, sq.seq, kvh, i);
    evict_one(a.pool, a.hkv, ptab[i / PAGE], kvh, i, xv, codes, meta);
  }
}

hipError_t launch_evict(const EvictArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_evict, dim3(a.hkv, a.n_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------------ decode-step write
// Grid (KV heads, sequences of the chunk); 256 threads (step_write_block).
__global__ __launch_bounds__(256) void k_step_write(StepArgs a) { step_write_block(a, blockIdx.x, blockIdx.y); }

hipError_t launch_step_write(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_step_write, dim3(a.hkv, a.n_seqs), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oscar
