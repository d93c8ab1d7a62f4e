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
#include "step_write.h"

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
// Grid (groups of tiles_per_wg tiles of 64 positions, KV heads, sequences of this chunk); 256
// threads.  Tile i covers positions len0 + 64 i ... of its sequence.  For a sequence that was
// empty, tile i >= 1 holds INT2 indices 64 (i-1) ... = page i-1.  launch_write sizes the groups
// so that all work-groups are resident at once (one residency round: no partial last round).
//
// Rotation on the matrix cores, transposed: x^T = R^T k^T with v_mfma_f32_16x16x32_f16.  The
// A operand is S R^T (S = 2^14) as two fp16 terms r0 = fp16(S R^T), r1 = fp16(S R^T - r0), so
// |S R^T - r0 - r1| <= 2^-22 |S R^T| (the scale keeps r1 out of the fp16 denormals); the B
// operand is the key row scaled by a power of two 2^sh that brings its largest magnitude into
// [2^14, 2^15), which makes the bf16 -> fp16 conversion exact; the products are exact in fp32 and
// accumulate in fp32; the result is multiplied by 2^-sh / S (exact).  The rotated key is then
// within about 2^-21 of sum_i |k_i R_ij| of the exact product, close to an fp32 dot product
// (bf16 terms, 2^-16, moved the quantizer input enough to flip ring-key roundings and INT2 codes
// measurably).  Wave w owns output channels 32 w .. 32 w + 31 and keeps its R^T operands in
// registers for all tiles of the work-group.

constexpr int XS = D + 4;  // fp32 row stride of the rotated tile (16-byte aligned rows)
constexpr int KS = D + 8;  // 16-bit row stride of the key / value tile
constexpr float ROT_TERM_SCALE = 16384.0f;  // S: the fp16 terms hold S R^T

typedef _Float16 v8h_w __attribute__((ext_vector_type(8)));
typedef unsigned short v2us_w __attribute__((ext_vector_type(2)));
typedef float v4f_w __attribute__((ext_vector_type(4)));
typedef unsigned int v4u_w __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256, 3) void k_write(WriteArgs a) {
  const int kvh = blockIdx.y, sl = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q4 = lane >> 4, n16 = lane & 15;
  const WriteSeq sq = a.seqs[sl];
  const int n_tiles = (a.n_new + PAGE - 1) / PAGE;
  const int tile0 = blockIdx.x * a.tiles_per_wg;
  if (tile0 >= n_tiles) return;
  const int tile1 = min(tile0 + a.tiles_per_wg, n_tiles);
  const int len = sq.len0 + a.n_new;
  const int n_int2 = (sq.len0 == 0) ? max(0, len - RING) : 0;  // INT2 tokens of this call

  // The tile buffer holds the scaled fp16 keys (rotation input), then the bf16 values (quantizer
  // input).
  __shared__ uint16_t tin[PAGE][KS];
  __shared__ int kshift[PAGE];             // per key row of the tile: its fp16 scale exponent sh
  __shared__ float x[PAGE][XS];            // rotated keys, fp32
  // quantizer parameters per (token, K/V group 2 isv + g): fp32 minimum and reciprocal scale
  __shared__ float qlo[PAGE][4], qinv[PAGE][4];

  // A operands: S R^T rows of this wave's output channels, 4 K-steps of 32 input channels, 2 terms
  const uint16_t* terms = reinterpret_cast<const uint16_t*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES + D * D * 4);
  v8h_w aop[2][4][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        aop[mt][ks][t] = *reinterpret_cast<const v8h_w*>(terms + t * D * D + (32 * wave + 16 * mt + n16) * D + 32 * ks + 8 * q4);

  const size_t row = static_cast<size_t>(a.hkv) * D;
  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  // A 64 x 128 bf16 tile (keys or values) moves global -> registers (16 bytes per thread and
  // step) -> LDS.  The inputs are read once and the INT2 pages are not read back by this launch,
  // so both go with the non-temporal hint (≈ 1 % faster than plain loads and stores).  The loads of the next tile are issued as soon as the registers have been
  // stored, so they are in flight while this tile is rotated and quantized.  Loads are never
  // conditional (rows past the call's tokens re-read the last row and are zeroed when stored;
  // past the work-group's last tile the last tile is read again), which keeps the compiler's
  // wait on them a counted one instead of a full drain.
  auto issue = [&](const uint16_t* base, int t, v4u_w* w) {
    const int nh = min(PAGE, a.n_new - t * PAGE);
    const uint16_t* src = base + (static_cast<size_t>(sq.src) * a.n_new + static_cast<size_t>(t) * PAGE) * row + kvh * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + 256 * r, j = min(i >> 4, nh - 1), c8 = i & 15;
      w[r] = __builtin_nontemporal_load(reinterpret_cast<const v4u_w*>(src + static_cast<size_t>(j) * row + 8 * c8));
    }
  };
  // Register -> LDS.  The rows past the call's tokens are then overwritten with zeros (LDS stores
  // only: selecting in registers let the compiler hoist the select, and with it the wait on the
  // loads, above the rotation).
  auto stash_tail = [&](int nh) {
    if (nh < PAGE) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = tid + 256 * r;
        if ((i >> 4) >= nh) *reinterpret_cast<v4u_w*>(&tin[i >> 4][8 * (i & 15)]) = v4u_w{0u, 0u, 0u, 0u};
      }
    }
  };
  auto stash = [&](int nh, const v4u_w* w) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + 256 * r;
      *reinterpret_cast<v4u_w*>(&tin[i >> 4][8 * (i & 15)]) = w[r];
    }
    stash_tail(nh);
  };
  // Keys go to LDS as fp16, each row (token) scaled by the power of two 2^sh that puts its largest
  // magnitude in [2^14, 2^15): exact, since a bf16 value has 8 significant bits and every entry
  // within 2^-28 of the row's largest is then an fp16 normal; smaller ones round to the fp16
  // denormal grid, an error below 2^-39 of the row's largest.  The conversion happens once, in
  // the registers the tile was loaded into, before they go to LDS: the 16 threads of a row take
  // the largest magnitude of their 8 values with packed 16-bit maxima, then combine them with
  // DPP row operations (xor 1, xor 2, half-row mirror, row mirror).  sh goes to LDS per row.
  auto stash_keys = [&](int nh, v4u_w* w) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = tid + 256 * r, j = i >> 4;
      v2us_w m2 = __builtin_bit_cast(v2us_w, w[r][0] & 0x7FFF7FFFu);
#pragma unroll
      for (int e = 1; e < 4; ++e) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(v2us_w, w[r][e] & 0x7FFF7FFFu));
      uint32_t mb = max(static_cast<uint32_t>(m2.x), static_cast<uint32_t>(m2.y));
      mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mb), 0xB1, 0xF, 0xF, false)));
      mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mb), 0x4E, 0xF, 0xF, false)));
      mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mb), 0x141, 0xF, 0xF, false)));
      mb = max(mb, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(mb), 0x140, 0xF, 0xF, false)));
      // exponent of the largest magnitude (bf16 exponent field, bias 127); all-zero rows keep 0
      const int ex = (mb >= 0x0080u) ? static_cast<int>(mb >> 7) - 127 : (mb ? -126 : 14);
      const int sh = 14 - ex;
      if ((i & 15) == 0) kshift[j] = sh;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t u = w[r][e];
        const _Float16 h0 = static_cast<_Float16>(__builtin_ldexpf(__uint_as_float(u << 16), sh));
        const _Float16 h1 = static_cast<_Float16>(__builtin_ldexpf(__uint_as_float(u & 0xFFFF0000u), sh));
        w[r][e] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                  (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
      }
    }
    stash(nh, w);
  };
  // page ids through the scalar cache (the table is not written by this kernel)
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)(a.page_table + static_cast<size_t>(sq.seq) * a.max_pages);
  v4u_w kreg[4], vreg[4];
  issue(a.k, tile0, kreg);
  issue(a.v, tile0, vreg);
  for (int tile = tile0; tile < tile1; ++tile) {
    const int n_here = min(PAGE, a.n_new - tile * PAGE);
    const int p0 = sq.len0 + tile * PAGE;
    const int next = min(tile + 1, tile1 - 1);
    // INT2 destination: tokens j with SINK <= p0 + j < SINK + n_int2 (tile >= 1 of an empty
    // sequence).  Only such a tile reads a page id, so the reads stay within the row's first
    // ceil(n_int2 / 64) entries (tiles holding window tokens only read nothing); fetched before
    // the tile's work.
    int n_q = 0;
    if (n_int2 > 0 && p0 >= SINK) n_q = max(0, min(n_here, SINK + n_int2 - p0));
    const int page = (n_q > 0) ? ptab[tile - 1] : 0;
    stash_keys(n_here, kreg);
    issue(a.k, next, kreg);
    __syncthreads();

    // rotation: 16-token column tiles; each (output tile, K-step) takes the two S R^T terms; the
    // accumulators of token 16 nt + n16 are unscaled by that row's 2^-sh / S
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      v8h_w b[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) b[ks] = *reinterpret_cast<const v8h_w*>(&tin[16 * nt + n16][32 * ks + 8 * q4]);
      const float sc = __builtin_ldexpf(1.0f / ROT_TERM_SCALE, -kshift[16 * nt + n16]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        v4f_w acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int t = 1; t >= 0; --t) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[mt][ks][t], b[ks], acc, 0, 0, 0);
        *reinterpret_cast<v4f_w*>(&x[16 * nt + n16][32 * wave + 16 * mt + 4 * q4]) = acc * sc;
      }
    }
    __syncthreads();
    stash(n_here, vreg);
    issue(a.v, next, vreg);
    __syncthreads();

    // BF16 destinations: sink / window (tiles holding such positions only)
    const bool any_bf16 = (p0 < SINK) || (p0 + n_here > SINK + n_int2);
    if (any_bf16) {
      // 8 channels of one token per thread and step, a fixed number of steps (a loop of unknown
      // trip count around the stores would make every later wait on the prefetch a full drain)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the thread index passes through an empty asm so that the compiler derives these
        // addresses here instead of keeping them live across the loop (they spilled)
        int t_ = tid;
        asm volatile("" : "+v"(t_));
        const int i = t_ + 256 * r, j = i >> 4, c8 = 8 * (i & 15), p = p0 + j;
        const bool int2 = (p >= SINK) && (p < SINK + n_int2);
        if (j < n_here && !int2) {
          const int slot = (p < SINK) ? p : SINK + (p - SINK) % WIN;
          const v4f_w x0 = *reinterpret_cast<const v4f_w*>(&x[j][c8]);
          const v4f_w x1 = *reinterpret_cast<const v4f_w*>(&x[j][c8 + 4]);
          const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          v4u_w kw;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            kw[e] = static_cast<uint32_t>(f32_to_bf16(xs[2 * e])) | (static_cast<uint32_t>(f32_to_bf16(xs[2 * e + 1])) << 16);
          *reinterpret_cast<v4u_w*>(a.ring + ring_head + static_cast<size_t>(slot) * D + c8) = kw;
          *reinterpret_cast<v4u_w*>(a.ring + ring_head + static_cast<size_t>(RING + slot) * D + c8) =
              *reinterpret_cast<const v4u_w*>(&tin[j][c8]);
        }
      }
    }

    if (n_q > 0) {  // uniform across the block
      uint32_t* blk = reinterpret_cast<uint32_t*>(a.pool + (static_cast<size_t>(page) * a.hkv + kvh) * HEAD_BLOCK);
      // ranges and parameters: one (token j, group g) per thread, waves 0-1 keys, waves 2-3 values.
      // The group's 64 values are read in 16-byte pieces; rows of consecutive lanes fall in
      // distinct banks.
      {
        int t_ = tid;                 // opaque copy: keeps these LDS addresses out of the loop's
        asm volatile("" : "+v"(t_));  // live registers (they spilled when hoisted)
        const int j = t_ & 63, g = (t_ >> 6) & 1, isv = t_ >> 7;
        float lo = 0.0f, inv = 0.0f;
        uint32_t mword = 0u;
        if (j < n_q) {
          float mn = INFINITY, mx = -INFINITY;
          if (isv) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const v4u_w w = *reinterpret_cast<const v4u_w*>(&tin[j][64 * g + 8 * i]);
              const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float v0 = __uint_as_float(ww[e] << 16), v1 = __uint_as_float(ww[e] & 0xFFFF0000u);
                mn = fminf(mn, fminf(v0, v1));
                mx = fmaxf(mx, fmaxf(v0, v1));
              }
            }
          } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const v4f_w v = *reinterpret_cast<const v4f_w*>(&x[j][64 * g + 4 * i]);
              mn = fminf(fminf(mn, v.x), fminf(v.y, fminf(v.z, v.w)));
              mx = fmaxf(fmaxf(mx, v.x), fmaxf(v.y, fmaxf(v.z, v.w)));
            }
          }
          const QParams qp = quant_params(mn, mx, isv ? C_V : C_K);
          lo = qp.lo;
          inv = qp.inv;  // 0 when the stored scale is 0: every code is then 0
          mword = static_cast<uint32_t>(qp.s16) | (static_cast<uint32_t>(qp.lo16) << 16);
        }
        // slots without a token: minimum 0, reciprocal scale 0 -> code 0, metadata 0
        __builtin_nontemporal_store(mword, &blk[(META_OFF >> 2) + 4 * j + 2 * isv + g]);
        qlo[j][2 * isv + g] = lo;
        qinv[j][2 * isv + g] = inv;
      }
      __syncthreads();
      // key words (inverse of kc_word): 16 channels 64 g + 16 kq + u of one token per word
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int w = tid + 256 * r;
        const int t2 = w >> 8, ln = (w & 255) >> 2, d = w & 3;
        const int t = 2 * t2 + (d >> 1), g = d & 1, kq = ln >> 4, n = ln & 15;
        const int j = 16 * t + n;
        QParams qp;
        qp.lo = qlo[j][g];
        qp.inv = qinv[j][g];
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4f_w v = *reinterpret_cast<const v4f_w*>(&x[j][64 * g + 16 * kq + 4 * i]);
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) word |= quant_code(vv[e], qp) << kc_bit(4 * i + e);
        }
        __builtin_nontemporal_store(word, &blk[(KC_OFF >> 2) + w]);
      }
      // value words (inverse of vc_word): 16 tokens of one channel per word
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int w = tid + 256 * r;
        const int ct = 4 * (w >> 8) + (w & 3), ln = (w & 255) >> 2;
        const int kq = ln >> 4, n = ln & 15, c = 16 * ct + n, gv = c >> 6;
        uint32_t word = 0;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const int jj = 32 * s2 + 8 * kq + kk;
            QParams qp;
            qp.lo = qlo[jj][2 + gv];
            qp.inv = qinv[jj][2 + gv];
            word |= quant_code(bf16_to_f32(tin[jj][c]), qp) << vc_bit(jj);
          }
        __builtin_nontemporal_store(word, &blk[(VC_OFF >> 2) + w]);
      }
    }
    __syncthreads();  // the next tile overwrites the tile buffer and the parameters
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_write, 256, 0) != hipSuccess) return 0;
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
  hipLaunchKernelGGL(k_write, dim3(groups, a.hkv, a.n_seqs), dim3(256), 0, s, a);
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
// Grid (KV heads, sequences); 256 threads.  Tokens are evicted one after the other.
__global__ __launch_bounds__(256) void k_evict(EvictArgs a) {
  const int kvh = blockIdx.x, sl = blockIdx.y;
  const EvictSeq sq = a.seqs[sl];
  __shared__ uint8_t codes[2][D];
  __shared__ uint16_t meta[8];
  for (int e = 0; e < a.n_evict; ++e)
    evict_one(a.pool, a.ring, a.page_table, a.hkv, a.max_pages, sq.seq, kvh, sq.n_int2 + e, codes, meta);
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
