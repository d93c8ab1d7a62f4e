// Fused INT2 decode attention on the gfx950 matrix cores.
//
// Method: axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy
// barrier", section "어텐션 통계 기반 회전과 Triton 커널의 결합" - the read path
// unpacks the INT2 bytes, dequantizes, handles the rotation and attends in one
// pass without extra memory traffic.  Here the rotation is applied once to the
// query (q' = q R_K; scores are unchanged because R_K is orthogonal) and the
// dequantization is folded into the matrix products:
//
//   score_j = sum_g s_jg (q'_g . c_jg) + lo_jg sum(q'_g)
//   out     = sum_j p_j (lo_jg + s_jg c_j) = sum_j p_j lo_jg + sum_j (p_j s_jg) c_j
//
// so both products run on the raw 2-bit codes:
//   * Q.K: i8 MFMA 16x16x64.  q' is split into two int8 terms (q' ~ sigma (t1 + t2/128),
//     error <= sigma/256) and the 16 A rows are (term, group, head): one instruction
//     per (16-token tile, channel group) covers 4 heads, both terms and both groups;
//     accumulation is exact integer arithmetic.  The rows are merged across lanes
//     with permlane swaps so that afterwards lane = token, register = head.
//   * P.V: f16 MFMA 16x16x32.  A value code c placed in mantissa bits e..e+1 of an
//     f16 with zero exponent *is* the f16 denormal c * 2^(e-24); one mask gives two
//     such operands per 32-bit word.  The per-position factor is folded into P
//     (A operand = p * s * 2^(4-e-LAZY), at most 65504 since p <= 2^LAZY), so the product
//     is exactly p s c 2^-(20+LAZY).  P is carried as an fp16 pair hi + lo (lo = the rounding
//     residual), which keeps 22 bits of p * s: the output is a strongly cancelling
//     sum, and a single fp16 P costs ~5e-4 relative error.  With GQA <= 4 the lo rows
//     ride in the otherwise empty rows 8..15 of the same instruction.
// Each wavefront walks the pages of one (sequence, KV head, split) with 128-bit loads
// of the raw page block, keeps a lazy running softmax maximum (rescaling only when a score
// exceeds it by more than 2^LAZY), and writes an (m, l, o) partial for the split combine.
#include <type_traits>

#include "common.h"
#include "step_write.h"

namespace oscar {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ workspace layout
// Per (sequence of the chunk, KV head): prepared query operands.
constexpr int QP_AOPS = 0;        // int8 A operands: [head block][lane][K-step][16 B] = 2 x 64 x 32 B
constexpr int QP_QF = 4096;       // fp32 q' (scaled to log2 units) [head][128]
constexpr int QP_CONST = 8192;    // fp32 per head: c_h = sigma_h / 128, Qt0'' , Qt1''
constexpr int QP_STRIDE = QPREP_STRIDE;

// Work sharing between the INT2 splits of one (sequence, KV head): the unit's full pages are
// cut into groups of share_group<G>() pages, one group per step of the page loop.  Work-group
// s starts on groups s and n_splits + s; every further group is handed out through one
// counter per unit (set to 2 n_splits by the query preparation) by an atomic that a step
// issues before its page loads and reads after its math, so the atomic returns while the step
// runs.  All splits of the unit share the query and their records are merged by the same
// softmax combine, so a record may cover any subset of the unit's pages; a work-group that the
// hardware packs onto a busy SIMD, or starts late, simply ends up with fewer groups.  Every
// step issues the same memory operations (the wait counts of the loop stay exact).  With
// DecodeArgs::share = 0 (the deterministic mode) split s covers the fixed range
// [s pps, min((s + 1) pps, full pages)) and its atomics add nothing.  A partially filled last
// page, and the BF16 sink + window work when it is folded, belong to split 0 and are done
// before its page loop.
template <int G>
__host__ __device__ constexpr int share_group() { return 3; }

// ------------------------------------------------------------------ query preparation
// One (KV head, sequence of the chunk, head block of up to 4 query heads) per 256-thread
// work-group: GQA 8 takes two work-groups per unit, each with the operands of its head block.
template <int G>
__host__ __device__ constexpr int qprep_heads() { return G < 4 ? G : 4; }
template <int G>
__device__ inline void qprep_block(const DecodeArgs& a, int kvh, int sl, int hb) {
  constexpr int GB = qprep_heads<G>();
  const int tid = threadIdx.x;
  const DecodeSeq sq = a.seqs[sl];
  __shared__ float qf[GB][D];
  __shared__ float sig[GB], rsig[GB];
  __shared__ float qt[GB][2];
  const float* rot = reinterpret_cast<const float*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES);
  const uint16_t* q = a.q + (static_cast<size_t>(sq.src) * a.hq + static_cast<size_t>(kvh) * G + 4 * hb) * D;
  uint8_t* ws = reinterpret_cast<uint8_t*>(a.part) + qprep_offset(a) + (static_cast<size_t>(sl) * a.hkv + kvh) * QP_STRIDE;
  // q' = q R: thread (half, c) reads column c of rows [64 half, 64 half + 64) once (coalesced)
  // for the block's heads; its 64 loads are issued before the query is staged, so the two
  // latencies overlap; the two halves are added through LDS
  const int c = tid & (D - 1), half = tid >> 7;
  float rcol[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) rcol[i] = rot[(64 * half + i) * D + c];
  __shared__ float qin[GB][D];
  for (int idx = tid; idx < GB * D; idx += 256) qin[idx / D][idx % D] = bf16_to_f32(q[idx]);
  __syncthreads();
  {
    __shared__ float part[2][GB][D];
    float acc[GB];
#pragma unroll
    for (int h = 0; h < GB; ++h) acc[h] = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i)
#pragma unroll
      for (int h = 0; h < GB; ++h) acc[h] = fmaf(qin[h][64 * half + i], rcol[i], acc[h]);
#pragma unroll
    for (int h = 0; h < GB; ++h) part[half][h][c] = acc[h];
    __syncthreads();
    for (int idx = tid; idx < GB * D; idx += 256) {
      const int h = idx / D, cc = idx % D;
      qf[h][cc] = (part[0][h][cc] + part[1][h][cc]) * a.scale_log2;
    }
  }
  __syncthreads();
  if ((tid >> 6) < GB) {
    // one wave per head: sigma = max|q'| / 127, per-group sums
    const int h = tid >> 6, l = tid & 63;
    float mx = fmaxf(fabsf(qf[h][l]), fabsf(qf[h][l + 64]));
    float s0 = qf[h][l], s1 = qf[h][l + 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off, 64));
      s0 += __shfl_xor(s0, off, 64);
      s1 += __shfl_xor(s1, off, 64);
    }
    if (l == 0) {
      sig[h] = (mx > 0.0f) ? mx / 127.0f : 1.0f;
      rsig[h] = (mx > 0.0f) ? 127.0f / mx : 1.0f;
      qt[h][0] = s0;
      qt[h][1] = s1;
    }
  }
  __syncthreads();
  float* wf = reinterpret_cast<float*>(ws + QP_QF) + 4 * hb * D;
  for (int idx = tid; idx < GB * D; idx += 256) wf[idx] = qf[idx / D][idx % D];
  float* wc = reinterpret_cast<float*>(ws + QP_CONST) + 3 * 4 * hb;
  if (tid < GB) {
    wc[3 * tid + 0] = sig[tid] / 128.0f;
    wc[3 * tid + 1] = qt[tid][0] * 128.0f / sig[tid];
    wc[3 * tid + 2] = qt[tid][1] * 128.0f / sig[tid];
  }
  // group counter of the unit: the first two groups of every split are taken
  int32_t* ctr = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(a.part) + counter_offset(a)) +
                 (static_cast<size_t>(sl) * a.hkv + kvh) * a.n_split_max;
  if (hb == 0 && tid == 0) ctr[0] = 2 * int2_splits(sq.n_int2, a.pages_per_split);
  // A operands, 2048 bytes: lane l, K-step g (channels 64 g + 16 (l / 16) + j, j = 0..15 = byte
  // j of the lane's 16 bytes); word w holds bytes j = 4 (w % 4) .. 4 (w % 4) + 3 of
  // (g, l) = ((w / 4) % 2, w / 8), four channels of one row m = l % 16.
  //   GQA <= 4: m = 4 (2 tau + grp) + h (rows of the other group's channels are zero); thread t
  //   builds words t and t + 256.
  //   GQA 8: m = 8 tau + h over the unit's 8 heads, both K-steps of every row non-zero (the
  //   split kernel keeps one accumulator per group); head block hb builds the 256 words of its
  //   heads' rows (bit 2 of l, bit 5 of w, equal to hb).
  uint32_t* wa = reinterpret_cast<uint32_t*>(ws + QP_AOPS);
#pragma unroll
  for (int r = 0; r < (G == 8 ? 1 : 2); ++r) {
    const int w = (G == 8) ? (((tid >> 5) << 6) | (hb << 5) | (tid & 31)) : tid + 256 * r;
    const int g = (w >> 2) & 1, l = w >> 3;
    const int m = l & 15, tau = m >> 3;
    const int grp = (G == 8) ? g : (m >> 2) & 1;
    const int h = m & 3;   // head within the block (GQA 8: block (m >> 2) & 1 = hb)
    uint32_t word = 0u;
    if (grp == g && h < GB) {
      const int c0 = 64 * g + 16 * (l >> 4) + 4 * (w & 3);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float x = qf[h][c0 + b] * rsig[h];
        const float t1 = rintf(x);
        const int v = static_cast<int>(tau == 0 ? t1 : rintf((x - t1) * 128.0f));
        word |= (static_cast<uint32_t>(v) & 0xFFu) << (8 * b);
      }
    }
    wa[w] = word;
  }
}

// Grid (KV heads, sequences of the chunk, head blocks), 256 threads.
template <int G>
__global__ __launch_bounds__(256) void k_qprep(DecodeArgs a) { qprep_block<G>(a, blockIdx.x, blockIdx.y, blockIdx.z); }

// The decode step's write and the query preparation in one launch: grid (KV heads, sequences,
// 1 + head blocks), z = 0 the write of one (KV head, sequence), z >= 1 the query preparation of
// head block z - 1.  The two touch disjoint memory (ring and pool; query, workspace), so they
// run side by side.  The write lands in the ring before the split kernel, which runs after this
// launch on the same stream, reads it (the new token attends to itself).
template <int G>
__global__ __launch_bounds__(256) void k_step_qprep(StepArgs w, DecodeArgs a) {
  if (blockIdx.z == 0) step_write_block(w, blockIdx.x, blockIdx.y);
  else qprep_block<G>(a, blockIdx.x, blockIdx.y, blockIdx.z - 1);
}

// ------------------------------------------------------------------ helpers

__device__ inline float lane_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ inline float lane_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// pointer into the global address space (loads through it are global, not flat, loads)
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;

__device__ inline v8h as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  v4u u = {a, b, c, d};
  return __builtin_bit_cast(v8h, u);
}

// Lazy running maximum: a page only triggers the rescale when one of its scores exceeds the
// running maximum by more than LAZY (log2 units).  Any reference value m gives the same
// softmax once the partials are combined (the record carries m), so the maximum only has to
// bound the exponentials: p = 2^(score - m) <= 2^LAZY, which the fp32 sums and the scaled
// fp16 P operand absorb.  On random-key workloads the running maximum of a 150-page split rises
// on about 11 % of the pages, by more than 2 on about 1 % (mostly the split's first page).
constexpr int LAZY = 2;


// Exponent e of the f16 denormal a value code lands in, by its position p' = 4 s + kk/2
// within the 32-bit word (see the unpack in the page loop).
__device__ inline int vcode_exp(int p) {
  constexpr int E[8] = {4, 6, 4, 6, 8, 4, 6, 8};
  return E[p];
}

// ------------------------------------------------------------------ BF16 sink + window split
// One wavefront over 64-slot chunks [ch0, ch1) of the ring (a range without any token writes the
// empty record m = -inf, l = 0, o = 0).  Scores: lane = ring slot, the lane reads its own key
// row in batches of KB 16-byte pieces.  Value product: lane = channel pair, token rows read in
// batches of VB = 32, so a chunk's values take two memory round trips (with batches of 8 the
// chunk's round trips made the BF16 work-groups the last to finish on the 8 x 32768-token
// layer).  Slots that hold no token are masked by a wave-uniform ballot; their (possibly
// uninitialised) rows never reach the sums.
template <int G>
__device__ inline void bf16_split(const DecodeArgs& a, const DecodeSeq& sq, int kvh, int sl, int split, int ch0, int ch1,
                           const float* qf, float (*pbuf)[64]) {
  constexpr int KB = (G == 8) ? 4 : 8;    // key pieces in flight per lane
  constexpr int VB = 32;                 // value rows in flight
  static_assert(64 % VB == 0 && VB < 64, "the row mask below shifts 1 by VB bits of a 64-bit word");
  const int lane = threadIdx.x;
  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  const uint16_t* kring = a.ring + ring_head;
  const uint16_t* vring = kring + static_cast<size_t>(RING) * D;
  const int n_win = max(0, sq.len - SINK - sq.n_int2);
  const int n_sink = min(sq.len, SINK);
  const int wfirst = sq.n_int2 % WIN;     // window position of the oldest window token
  float m[G], l[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m[h] = -INFINITY; l[h] = 0.0f; o0[h] = 0.0f; o1[h] = 0.0f; }
  for (int ch = ch0; ch < ch1; ++ch) {
    const int slot = ch * 64 + lane;
    const bool ok = (slot < SINK) ? (slot < n_sink) : (((slot - SINK - wfirst + WIN) % WIN) < n_win);
    const uint64_t okmask = __ballot(ok);
    if (okmask == 0) continue;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.0f;
    const uint4* kr = reinterpret_cast<const uint4*>(kring + static_cast<size_t>(slot) * D);
#pragma unroll 1
    for (int c0 = 0; c0 < D / 8; c0 += KB) {
      uint4 w[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) w[i] = kr[c0 + i];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const uint32_t ww[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(ww[e] << 16), k1 = __uint_as_float(ww[e] & 0xFFFF0000u);
          const int c = 8 * (c0 + i) + 2 * e;
#pragma unroll
          for (int h = 0; h < G; ++h) s[h] = fmaf(qf[h * D + c + 1], k1, fmaf(qf[h * D + c], k0, s[h]));
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sc = ok ? s[h] : -INFINITY;
      const float mn = fmaxf(m[h], lane_max(sc));
      const float alpha = (m[h] == -INFINITY) ? 0.0f : exp2f(m[h] - mn);
      const float p = ok ? exp2f(sc - mn) : 0.0f;
      l[h] = l[h] * alpha + lane_sum(p);
      o0[h] *= alpha;
      o1[h] *= alpha;
      m[h] = mn;
      pbuf[h][lane] = p;
    }
    __syncthreads();
    // value product: lane owns channels 2 lane, 2 lane + 1
    const uint32_t* vr = reinterpret_cast<const uint32_t*>(vring + static_cast<size_t>(ch * 64) * D) + lane;
#pragma unroll 1
    for (int j0 = 0; j0 < 64; j0 += VB) {
      if (((okmask >> j0) & ((1ull << VB) - 1)) == 0) continue;  // wave-uniform
      uint32_t w[VB];
#pragma unroll
      for (int j = 0; j < VB; ++j) w[j] = vr[(j0 + j) * (D / 2)];
#pragma unroll
      for (int j = 0; j < VB; ++j) {
        const bool okj = (okmask >> (j0 + j)) & 1;
        const float v0 = okj ? __uint_as_float(w[j] << 16) : 0.0f;
        const float v1 = okj ? __uint_as_float(w[j] & 0xFFFF0000u) : 0.0f;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          o0[h] = fmaf(pbuf[h][j0 + j], v0, o0[h]);
          o1[h] = fmaf(pbuf[h][j0 + j], v1, o1[h]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* rec = a.part + ((static_cast<size_t>(sl) * a.hq + kvh * G + h) * a.n_split_max + split) * PART_STRIDE;
    if (lane == 0) { rec[0] = m[h]; rec[1] = l[h]; }
    rec[2 + 2 * lane] = o0[h];
    rec[3 + 2 * lane] = o1[h];
  }
}

// ------------------------------------------------------------------ INT2 page loop
// Grid (KV heads x sequences of the chunk, splits), one wavefront per work-group.  Work-groups
// are dispatched split by split, so every unit gets one work-group of each dispatch age (waves
// of a SIMD issue oldest first, and with the unit slowest in the grid the units dispatched last
// finished up to 50 % after the first); within a split the units are rotated by the split index,
// so that with the dispatcher's round robin over the XCDs (linear index mod 8) the splits of a
// unit land on different XCDs (units confined to one XCD finished up to 30 % apart, with the
// XCDs' speeds).  The page sharing within a unit then evens out the rest.
// Records 0 .. n_isplits-1 are INT2 page ranges, record n_isplits the BF16 sink + window.

// The page work of INT2 split `split` of one unit, written to record `split`: split 0 first does
// the folded BF16 work and the partially filled last page.
template <int G>
__device__ __forceinline__ void int2_split(const DecodeArgs& a, int kvh, int sl, const DecodeSeq& sq, int split,
                                           bool fold, int n_isplits, float (*pbuf_bf)[64]) {
  constexpr int GP = G < 4 ? 4 : G;       // heads padded to a multiple of 4
  constexpr int HB = GP / 4;              // head blocks (MFMA row blocks of Q.K)
  const int lane = threadIdx.x, q4 = lane >> 4, n16 = lane & 15;
  const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.part) + qprep_offset(a) +
                      (static_cast<size_t>(sl) * a.hkv + kvh) * QP_STRIDE;
  // P operand staging, one MFMA row block (16 rows) per block of rows: GQA <= 4: hi rows
  // (group, head) 0..7, lo rows 8..15; GQA 8: per group g, rows 16 g + h (hi) and 16 g + 8 + h
  // (lo), so that each group's block meets only that group's 64 value channels
  __shared__ _Float16 plds[32][64];

  // ---- prologue: query operands (kept in LDS and read per page, which leaves the registers
  // for a third page buffer) and per-head constants
  __shared__ v4i aop_lds[2][64];   // [K-step][lane] (see qprep_block)
#pragma unroll
  for (int g = 0; g < 2; ++g)
    aop_lds[g][lane] = *reinterpret_cast<const v4i*>(ws + QP_AOPS + (lane * 2 + g) * 16);
  // per-head constants are wave-uniform: keep them in scalar registers
  float cst[G][3];
  const float* wc = reinterpret_cast<const float*>(ws + QP_CONST);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < 3; ++k)
      cst[h][k] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wc[3 * h + k])));
  for (int i = lane; i < 32 * 64; i += 64) (&plds[0][0])[i] = static_cast<_Float16>(0.0f);
  // staging rows of head h: hi and lo residual of groups 0 and 1 (see plds)
  constexpr int ROW_HI1 = (G == 8) ? 16 : GP, ROW_LO0 = 8, ROW_LO1 = (G == 8) ? 24 : 8 + GP;

  // token of this lane after the Q.K row merge (which pairs tiles 0/2 and 1/3): the lane index
  const int tok = lane;
  // the extra 2^-LAZY keeps p * s * pfac within fp16 range while p may reach 2^LAZY
  const float pfac = __builtin_ldexpf(1.0f, 4 - LAZY - vcode_exp(4 * (tok >> 5) + ((tok & 7) >> 1)));

  float m_run[G], l_acc[G], lo_acc[2][G];
#pragma unroll
  for (int h = 0; h < G; ++h) { m_run[h] = -INFINITY; l_acc[h] = 0.0f; lo_acc[0][h] = 0.0f; lo_acc[1][h] = 0.0f; }
  // P.V accumulators: rows (grp, h) = grp * GP + h (16 rows cover GQA <= 8), columns = channels
  v4f oacc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) oacc[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int first = split * a.pages_per_split;
  const int32_t* ptab = a.page_table + static_cast<size_t>(sq.seq) * a.max_pages;
  const size_t head_off = static_cast<size_t>(kvh) * HEAD_BLOCK;
  const size_t page_stride = static_cast<size_t>(a.hkv) * HEAD_BLOCK;
  __syncthreads();

  // Raw page block (128-bit loads): key codes (2 per lane), value codes (2 per lane), and the
  // metadata of this lane's token.  Pages are loaded ahead into rotating register sets, always
  // issuing the next load (clamped to the last page) so the wait counts stay exact.  Page ids
  // are scalar loads through the constant address space, fetched one page ahead: they wait on
  // the scalar/LDS counter, so no wait on the vector-memory counter ever drains the prefetch.
  struct Raw { v4u kc0, kc1, vc0, vc1, md; };
  const __attribute__((address_space(4))) int32_t* ptab_c =
      (const __attribute__((address_space(4))) int32_t*)(ptab);
  auto load_block = [&](int page, Raw& r) {
    // the page base is wave-uniform: pin it to scalar registers so that the compiler cannot
    // reassociate the lane offsets into loop-invariant 64-bit per-lane addresses
    uint64_t base = reinterpret_cast<uint64_t>(a.pool + static_cast<size_t>(page) * page_stride + head_off);
    asm volatile("" : "+s"(base));
    const gptr<uint8_t> blk = reinterpret_cast<gptr<uint8_t>>(base);
    const gptr<v4u> kp = reinterpret_cast<gptr<v4u>>(blk + KC_OFF) + lane;
    const gptr<v4u> vp = reinterpret_cast<gptr<v4u>>(blk + VC_OFF) + lane;
    r.kc0 = __builtin_nontemporal_load(kp);
    r.kc1 = __builtin_nontemporal_load(kp + 64);
    r.vc0 = __builtin_nontemporal_load(vp);
    r.vc1 = __builtin_nontemporal_load(vp + 64);
    // the metadata base past the immediate-offset range gets its own scalar pair
    uint64_t base_md = base + META_OFF;
    asm volatile("" : "+s"(base_md));
    r.md = __builtin_nontemporal_load(reinterpret_cast<gptr<v4u>>(base_md) + lane);  // token = lane
  };

  // FULL (a compile-time tag): every token of the page holds a code, so no per-token masking
  auto process_page = [&](int lp, const Raw& raw, auto full_tag) {
    constexpr bool FULL = decltype(full_tag)::value;
    const v4u& kc0 = raw.kc0;
    const v4u& kc1 = raw.kc1;
    const v4u& vc0 = raw.vc0;
    const v4u& vc1 = raw.vc1;
    const v4u& md = raw.md;
    const int n_valid = min(PAGE, sq.n_int2 - lp * PAGE);

    // ---- Q.K on the matrix cores, columns = tokens of tile t.  GQA <= 4: acc[0][t] rows
    // (tau, grp, h), the two K-steps (channel groups) summed, the other group's rows of each
    // K-step zero.  GQA 8: acc[g][t] rows (tau, h) of K-step g alone (one accumulator per group:
    // half the instructions of a row layout with a zero half).
    v4i acc[HB][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const v4u& kc = (t < 2) ? kc0 : kc1;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const uint32_t w = kc[2 * (t & 1) + g];
        const v4i b = {static_cast<int>(w & 0x03030303u), static_cast<int>((w >> 2) & 0x03030303u),
                       static_cast<int>((w >> 4) & 0x03030303u), static_cast<int>((w >> 6) & 0x03030303u)};
        if (G == 8) {
          acc[g][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop_lds[g][lane], b, v4i{0, 0, 0, 0}, 0, 0, 0);
        } else {
          if (g == 0) acc[0][t] = v4i{0, 0, 0, 0};
          acc[0][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop_lds[g][lane], b, acc[0][t], 0, 0, 0);
        }
      }
    }
    // ---- merge rows across lanes: afterwards lane = token, x0/x1 = group 0/1 dot per head.
    // Lane group q4 holds rows (tau, s) = (q4 / 2, q4 % 2), where s is the group (GQA <= 4) or
    // the head half (GQA 8).  The 32-lane swaps of tiles 0/2 and 1/3 put the tau = 0 rows of both
    // tiles of a pair in one register and the tau = 1 rows in the other (lanes 0-31 the first
    // tile, 32-63 the second); the two terms are merged in integers; the 16-lane swap then
    // separates s, leaving tiles 0, 1, 2, 3 in lanes 0-15, 16-31, 32-47, 48-63.
    float x0[GP], x1[GP];
#pragma unroll
    for (int a2 = 0; a2 < HB; ++a2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const auto s02 = __builtin_amdgcn_permlane32_swap(acc[a2][0][r], acc[a2][2][r], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(acc[a2][1][r], acc[a2][3][r], false, false);
        const int c02 = static_cast<int>((static_cast<uint32_t>(s02[0]) << 7) + static_cast<uint32_t>(s02[1]));
        const int c13 = static_cast<int>((static_cast<uint32_t>(s13[0]) << 7) + static_cast<uint32_t>(s13[1]));
        const auto gg = __builtin_amdgcn_permlane16_swap(c02, c13, false, false);
        const float s_even = static_cast<float>(static_cast<int>(gg[0]));
        const float s_odd = static_cast<float>(static_cast<int>(gg[1]));
        if (G == 8) {   // accumulator a2 = group, s = head half
          (a2 == 0 ? x0 : x1)[r] = s_even;
          (a2 == 0 ? x0 : x1)[4 + r] = s_odd;
        } else {        // s = group, head r
          x0[r] = s_even;
          x1[r] = s_odd;
        }
      }

    // ---- scores (log2 units) and the running max
    const float sk0 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.x & 0xFFFF)));
    const float lk0 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.x >> 16)));
    const float sk1 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.y & 0xFFFF)));
    const float lk1 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.y >> 16)));
    const bool valid = FULL || tok < n_valid;
    float z[G];
    float zmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float y = fmaf(lk1, cst[h][2], fmaf(lk0, cst[h][1], fmaf(sk1, x1[h], sk0 * x0[h])));
      // score minus the running maximum in one fused step (+inf while the maximum is -inf,
      // which sends the page through the rescale below)
      z[h] = valid ? fmaf(y, cst[h][0], -m_run[h]) : -INFINITY;
      zmax = fmaxf(zmax, z[h]);
      x0[h] = y;  // the unscaled dot, for the rescale path
    }
    if (__any(zmax > static_cast<float>(LAZY))) {
      // the running maximum is stale by more than 2^LAZY: move it to the exact maximum so far
      // and rescale everything accumulated (in practice only on a split's first page)
      float alpha[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sc = valid ? x0[h] * cst[h][0] : -INFINITY;
        const float mn = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
            __builtin_bit_cast(int, fmaxf(m_run[h], lane_max(sc)))));
        alpha[h] = (m_run[h] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[h] - mn);
        m_run[h] = mn;
        z[h] = sc - mn;
        l_acc[h] *= alpha[h];
        lo_acc[0][h] *= alpha[h];
        lo_acc[1][h] *= alpha[h];
      }
      // oacc row 4 q4 + r: G <= 4 -> head r; G = 8 -> head 4 (q4 % 2) + r (hi rows in lanes
      // 0-31, their lo residuals in lanes 32-63)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // values, not array elements, in the conditional: a conditional of two lvalues would
        // select an address and leave alpha[] in private memory
        const float a_lo = alpha[r % G], a_hi = alpha[(4 + r) % G];
        float al;
        if (G == 8) al = (q4 & 1) ? a_hi : a_lo;
        else al = (r < G) ? a_lo : 0.0f;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) oacc[ct][r] *= al;
      }
    }

    // ---- probabilities, row sums, minimum terms, and the P operand staging
    const float sv0 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.z & 0xFFFF)));
    const float lv0 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.z >> 16)));
    const float sv1 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.w & 0xFFFF)));
    const float lv1 = __half2float(__ushort_as_half(static_cast<unsigned short>(md.w >> 16)));
    const float f0 = sv0 * pfac, f1 = sv1 * pfac;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // z <= LAZY here; the raw exp2 flushes results below 2^-126 to zero, which is harmless
      const float p = valid ? __builtin_amdgcn_exp2f(z[h]) : 0.0f;
      l_acc[h] += p;
      lo_acc[0][h] = fmaf(p, lv0, lo_acc[0][h]);
      lo_acc[1][h] = fmaf(p, lv1, lo_acc[1][h]);
      const float a0 = p * f0, a1 = p * f1;
      const _Float16 h0 = static_cast<_Float16>(a0), h1 = static_cast<_Float16>(a1);
      plds[h][tok] = h0;
      plds[ROW_HI1 + h][tok] = h1;
      plds[ROW_LO0 + h][tok] = static_cast<_Float16>(a0 - static_cast<float>(h0));
      plds[ROW_LO1 + h][tok] = static_cast<_Float16>(a1 - static_cast<float>(h1));
    }
    __syncthreads();
    // A operand rows (grp, h) = lane % 16: tokens 32 s + 8 (lane / 16) + 0..7
    const v4u pa0 = *reinterpret_cast<const v4u*>(&plds[n16][8 * q4]);
    const v4u pa1 = *reinterpret_cast<const v4u*>(&plds[n16][32 + 8 * q4]);
    const v8h pA0 = __builtin_bit_cast(v8h, pa0), pA1 = __builtin_bit_cast(v8h, pa1);
    v8h pB0 = pA0, pB1 = pA1;
    if (G == 8) {
      pB0 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(&plds[16 + n16][8 * q4]));
      pB1 = __builtin_bit_cast(v8h, *reinterpret_cast<const v4u*>(&plds[16 + n16][32 + 8 * q4]));
    }
    __syncthreads();

    // ---- P.V on the matrix cores, value codes as f16 denormals
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const uint32_t w = (ct < 4) ? vc0[ct & 3] : vc1[ct & 3];
      const uint32_t lo4 = w << 4, hi6 = w >> 6;
      const v8h b0 = as_h8(lo4 & 0x00300030u, lo4 & 0x00C000C0u, w & 0x00300030u, w & 0x00C000C0u);
      const v8h b1 = as_h8(w & 0x03000300u, hi6 & 0x00300030u, hi6 & 0x00C000C0u, hi6 & 0x03000300u);
      // GQA 8: group 0's row block for channel tiles 0..3, group 1's for 4..7
      const v8h& xa0 = (G == 8 && ct >= 4) ? pB0 : pA0;
      const v8h& xa1 = (G == 8 && ct >= 4) ? pB1 : pA1;
      oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa0, b0, oacc[ct], 0, 0, 0);
      oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa1, b1, oacc[ct], 0, 0, 0);
    }
  };

  // split 0's extra work first: the BF16 sink + window records (when folded) and the partially
  // filled last page; then every vector-memory access has returned, so the page loop starts
  // from a clean wait state
  if (split == 0) {
    if (fold)
      bf16_split<G>(a, sq, kvh, sl, n_isplits, 0, RING_CHUNKS, reinterpret_cast<const float*>(ws + QP_QF), pbuf_bf);
    if (sq.n_int2 % PAGE != 0) {
      Raw b;
      load_block(ptab_c[sq.n_int2 / PAGE], b);
      process_page(sq.n_int2 / PAGE, b, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(0);
  }

  // ---- the page stream of this work-group (work sharing within the unit, see share_group):
  // groups of NB consecutive full pages, one group per loop step
  constexpr int NB = share_group<G>();      // rotating register sets = pages per step
  const int n_full = sq.n_int2 / PAGE;
  const int pps = a.pages_per_split;
  int32_t* ctr = reinterpret_cast<int32_t*>(reinterpret_cast<uint8_t*>(a.part) + counter_offset(a)) +
                 (static_cast<size_t>(sl) * a.hkv + kvh) * a.n_split_max;
  const int inc = a.share ? 1 : 0;
  int pend = 0;      // lane 0: the group index the step's claim returned
  auto claim = [&]() {
    int old = 0;
    if (lane == 0) {
      // a per-lane address for the compiler: a wave-uniform one would let it broadcast the
      // result right away (a full wait on the vector-memory counter)
      uint64_t p = reinterpret_cast<uint64_t>(ctr);
      asm volatile("" : "+v"(p));
      old = __hip_atomic_fetch_add(reinterpret_cast<__attribute__((address_space(1))) int32_t*>(p), inc,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    pend = old;
  };
  // a group: first page and page count (0: nothing left)
  auto group = [&](int g, int& g_first, int& g_n) {
    g_first = __builtin_amdgcn_readfirstlane(g * NB);
    g_n = __builtin_amdgcn_readfirstlane(max(0, min(NB, n_full - g * NB)));
  };
  const int own_end = min(first + pps, n_full);   // the deterministic mode's range
  int det_next = first + 2 * NB;
  // the group after the next one: the claimed group, or the next of the fixed range
  auto resolve = [&](int& g_first, int& g_n) {
    if (a.share) {
      group(__builtin_amdgcn_readfirstlane(pend), g_first, g_n);
    } else {
      g_first = det_next;
      g_n = max(0, min(NB, own_end - det_next));
      det_next += NB;
    }
  };
  int t_first, t_n, n_first, n_n;
  if (a.share) {
    group(split, t_first, t_n);
    group(n_isplits + split, n_first, n_n);
  } else {
    t_first = first;
    t_n = max(0, min(NB, own_end - first));
    n_first = first + NB;
    n_n = max(0, min(NB, own_end - first - NB));
  }
  // page ids of a group (a missing page repeats the previous id, so every step issues the same
  // loads and the wait counts stay exact); the third id is unused when NB = 2
  int last_id = ptab_c[(t_n > 0) ? t_first : 0];
  auto group_ids = [&](int g_first, int g_n, int& i0, int& i1, int& i2) {
    i0 = (g_n > 0) ? ptab_c[g_first] : last_id;
    i1 = (g_n > 1) ? ptab_c[g_first + 1] : i0;
    i2 = (NB > 2 && g_n > 2) ? ptab_c[g_first + 2] : i1;
    last_id = (NB > 2) ? i2 : i1;
  };
  int t0, t1, t2, n0, n1, n2;
  group_ids(t_first, t_n, t0, t1, t2);
  group_ids(n_first, n_n, n0, n1, n2);

  {
    // Three rotating register sets: two pages in flight while one is processed (GQA 8 too: at its
    // 2 waves per SIMD the third set fits the register budget; with one page in flight it was
    // 1.4 % slower).  One step processes the current group t and loads the next group n; the
    // loop has a single exit.
    const std::true_type full{};
    Raw b0, b1, b2;
    load_block(t0, b0);
    __builtin_amdgcn_sched_barrier(0);  // keep page order in the queue: waits stay vmcnt(10)
    load_block(t1, b1);
    __builtin_amdgcn_sched_barrier(0);
    if (t_n > 0) {
      do {
        claim();
        load_block(t2, b2);
        __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the page's math
        process_page(0, b0, full);
        load_block(n0, b0);
        __builtin_amdgcn_sched_barrier(0);
        if (t_n > 1) process_page(0, b1, full);
        load_block(n1, b1);
        __builtin_amdgcn_sched_barrier(0);
        if (t_n > 2) process_page(0, b2, full);
        t_n = n_n;
        t2 = n2;
        resolve(n_first, n_n);
        group_ids(n_first, n_n, n0, n1, n2);
      } while (t_n > 0);
    }
  }

  // ---- epilogue: reduce per-lane sums, write (m, l, o) partials
  float lsum[G], losum[2][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = lane_sum(l_acc[h]);
    losum[0][h] = lane_sum(lo_acc[0][h]);
    losum[1][h] = lane_sum(lo_acc[1][h]);
  }
  const float two20 = __builtin_ldexpf(1.0f, 20 + LAZY);  // undoes pfac's 2^(e - 4 + LAZY)
  // rows 8..15 (lanes 32..63) of every row block hold the lo-residual products of rows 0..7:
  // fold them in
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) oacc[ct][r] += __shfl_xor(oacc[ct][r], 32, 64);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* rec = a.part + ((static_cast<size_t>(sl) * a.hq + kvh * G + h) * a.n_split_max + split) * PART_STRIDE;
    if (lane == 0) { rec[0] = m_run[h]; rec[1] = lsum[h]; }
  }
  // oacc[ct] row 4 q4 + r (< 8) = grp * 4 + h for GQA <= 4, h for GQA 8 (whose row block of
  // channel tile ct is group ct / 4's); channel 16 ct + n16 belongs to group ct / 4
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    const int grp = ct >> 2;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q4 + r;
      int h;
      bool mine;
      if (GP == 4) { h = row - 4 * grp; mine = (row >> 2) == grp && h < G; }
      else { h = row; mine = row < 8; }
      if (mine) {
        float* rec = a.part + ((static_cast<size_t>(sl) * a.hq + kvh * G + (h % G)) * a.n_split_max + split) * PART_STRIDE;
        rec[2 + 16 * ct + n16] = fmaf(oacc[ct][r], two20, losum[grp][h % G]);
      }
    }
  }
}


template <int G>
// Occupancy target: 3 waves per SIMD (2 for GQA 8, whose P.V needs twice the operands).
__global__ __launch_bounds__(64, G == 8 ? 2 : 3) void k_decode_mfma(DecodeArgs a) {
  const int n_units = a.hkv * a.n_seqs;
  const int y = blockIdx.y;   // the unit's work-group index, in dispatch order
  const int unit = (static_cast<int>(blockIdx.x) + n_units - y % n_units) % n_units;
  const int kvh = unit % a.hkv, sl = unit / a.hkv;
  const int lane = threadIdx.x;
  const DecodeSeq sq = a.seqs[sl];
  const int n_isplits = int2_splits(sq.n_int2, a.pages_per_split);
  const int n_bsplits = bf16_splits(sq.n_int2, sq.len, a.pages_per_split, 0);
  // the BF16 sink + window tokens (partial records n_isplits ..) are done first by INT2 split 0
  // (the unit's oldest work-group) when the plan folds them, else by work-groups of their own,
  // dispatched before the INT2 splits: work-groups dispatched last issue last and would finish
  // last with work that nobody can share
  const bool fold = bf16_folded(sq.n_int2, sq.len, a.pages_per_split, 0);
  const int nbw = fold ? 0 : n_bsplits;
  if (y >= n_isplits + nbw) return;
  const int split = y - nbw;  // INT2 split; negative for a BF16 work-group

  __shared__ float pbuf_bf[G][64];
  if (split < 0) {
    const uint8_t* ws = reinterpret_cast<const uint8_t*>(a.part) + qprep_offset(a) +
                        (static_cast<size_t>(sl) * a.hkv + kvh) * QP_STRIDE;
    const int b = y;
    bf16_split<G>(a, sq, kvh, sl, n_isplits + b, (RING_CHUNKS * b) / n_bsplits, (RING_CHUNKS * (b + 1)) / n_bsplits,
                  reinterpret_cast<const float*>(ws + QP_QF), pbuf_bf);
    return;
  }
  int2_split<G>(a, kvh, sl, sq, split, fold, n_isplits, pbuf_bf);
}

// Work-groups to plan for one residency round: all wave slots of the device but one per
// compute unit.  Measured on the 100000-token, 32-sequence, 8-KV-head decode: work-groups that
// fill every slot (12 per CU) ran about 15% slower per page than 11 per CU.
template <typename K>
static int resident_for(K kernel, int block) {
  int dev = 0, n_cu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return 0;
  return n_cu * (per_cu > 1 ? per_cu - 1 : 1);
}

int decode_resident_workgroups(int gqa, int kernel) {
  static int cache[2][9] = {};
  const int k = kernel ? 1 : 0;
  if (gqa < 1 || gqa > 8) return 1024;
  if (cache[k][gqa] == 0) {
    int r = 0;
    if (k == 1) {
      r = 1024;  // reference kernel: 256 threads per work-group
    } else {
      switch (gqa) {
        case 1: r = resident_for(k_decode_mfma<1>, 64); break;
        case 2: r = resident_for(k_decode_mfma<2>, 64); break;
        case 4: r = resident_for(k_decode_mfma<4>, 64); break;
        case 8: r = resident_for(k_decode_mfma<8>, 64); break;
        default: r = 0;
      }
    }
    cache[k][gqa] = r > 0 ? r : 1024;
  }
  return cache[k][gqa];
}

template <int G>
static hipError_t launch_g(const StepArgs* w, const DecodeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int HB = (G + 3) / 4;   // query-preparation work-groups per unit
  if (w) hipLaunchKernelGGL(k_step_qprep<G>, dim3(a.hkv, a.n_seqs, 1 + HB), dim3(256), 0, s, *w, a);
  else hipLaunchKernelGGL(k_qprep<G>, dim3(a.hkv, a.n_seqs, HB), dim3(256), 0, s, a);
  if (t0) {
    const hipError_t e = hipEventRecord(t0, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_decode_mfma<G>, dim3(a.hkv * a.n_seqs, a.wg_rows), dim3(64), 0, s, a);
  if (t1) {
    const hipError_t e = hipEventRecord(t1, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const StepArgs* w, const DecodeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (w && (w->n_seqs != a.n_seqs || w->hkv != a.hkv)) return hipErrorInvalidValue;
  switch (a.hq / a.hkv) {
    case 1: return launch_g<1>(w, a, s, t0, t1);
    case 2: return launch_g<2>(w, a, s, t0, t1);
    case 4: return launch_g<4>(w, a, s, t0, t1);
    case 8: return launch_g<8>(w, a, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace oscar
