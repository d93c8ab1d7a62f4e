// Read path: split-K GQA decode attention over the mixed-precision paged cache,
// then the cross-split softmax combine.
//
// Method: axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy
// barrier", section "어텐션 통계 기반 회전과 Triton 커널의 결합" - the read path
// unpacks the INT2 bytes, dequantizes, handles the key rotation and attends in
// one fused pass with no extra memory traffic.  The rotation is handled on the
// query side: scores of the stored rotated keys against q' = q . R_K equal the
// unrotated scores because R_K is orthogonal.  Split-K over pages with an exact
// (m, l, o) merge is this library's work decomposition; the pages do not
// describe one.
#include <algorithm>

#include "common.h"

namespace oscar {

// ------------------------------------------------------------------ shared pieces

// q' = q . R_K for the GQA heads of one KV head, scaled into the log2 domain.
template <int GQA>
__device__ inline void rotate_queries(const DecodeArgs& a, const DecodeSeq& sq, int kvh, float (*qr)[D], int tid) {
  const float* rot = reinterpret_cast<const float*>(a.rot + static_cast<size_t>(kvh) * ROT_HEAD_BYTES);
  const uint16_t* q = a.q + (static_cast<size_t>(sq.src) * a.hq + static_cast<size_t>(kvh) * GQA) * D;
  for (int idx = tid; idx < GQA * D; idx += blockDim.x) {
    const int h = idx / D, c = idx % D;
    float acc = 0.0f;
    for (int i = 0; i < D; ++i) acc = fmaf(bf16_to_f32(q[h * D + i]), rot[i * D + c], acc);
    qr[h][c] = acc * a.scale_log2;
  }
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}


// Dequantize 64 tokens (keys, or values when vals) of one chunk into LDS and
// mark which of them exist.  BF16 chunk ch covers ring slots 64 ch .. 64 ch + 63.
__device__ inline void stage_chunk(const DecodeArgs& a, const DecodeSeq& sq, const uint8_t* blk,
                                   size_t ring_head, int ch, int n_win, int first, bool bf16_split,
                                   bool vals, float (*xd)[D + 1], uint8_t* valid, int tid) {
  if (bf16_split) {
    // Ring slots that hold no token contain whatever the caller's buffer held (possibly NaN):
    // they are zeroed here, since a zero probability times NaN is still NaN.
    const size_t base = ring_head + (vals ? static_cast<size_t>(RING) * D : 0);
    for (int i = tid; i < PAGE * D; i += 256) {
      const int j = i / D, c = i % D, slot = ch * PAGE + j;
      const bool ok = (slot < SINK) ? (slot < min(sq.len, SINK))
                                    : (((slot - SINK - (sq.n_int2 % WIN) + WIN) % WIN) < n_win);
      xd[j][c] = ok ? bf16_to_f32(a.ring[base + static_cast<size_t>(slot) * D + c]) : 0.0f;
      if (c == 0) valid[j] = ok;
    }
  } else {
    const uint32_t* kw = reinterpret_cast<const uint32_t*>(blk + (vals ? VC_OFF : KC_OFF));
    const __half* meta = reinterpret_cast<const __half*>(blk + META_OFF);
    for (int i = tid; i < PAGE * D; i += 256) {
      const int j = i / D, c = i % D, g = c >> 6;
      const bool ok = ((first + ch) * PAGE + j) < sq.n_int2;
      const uint32_t code = vals ? (kw[vc_word(j, c)] >> vc_bit(j)) & 3u : (kw[kc_word(j, c)] >> kc_bit(c)) & 3u;
      const int mo = 8 * j + (vals ? 4 : 0) + 2 * g;
      xd[j][c] = ok ? __half2float(meta[mo + 1]) + __half2float(meta[mo]) * static_cast<float>(code) : 0.0f;
      if (c == 0) valid[j] = ok;
    }
  }
}

// ------------------------------------------------------------------ reference-grade kernel
// Grid (splits, KV heads, sequences of this chunk), 256 threads.  Split s <
// n_int2_splits covers INT2 pages [s P, min((s+1) P, n_pages)); split
// n_int2_splits covers the BF16 sink + window ring (five 64-slot chunks).
// Every step is plain fp32 arithmetic on dequantized values.

template <int GQA>
__global__ __launch_bounds__(256) void k_decode_simple(DecodeArgs a) {
  const int split = blockIdx.x, kvh = blockIdx.y, sl = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const DecodeSeq sq = a.seqs[sl];
  const int n_pages = (sq.n_int2 + PAGE - 1) / PAGE;
  const int n_isplits = (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  if (split > n_isplits) return;
  const bool bf16_split = (split == n_isplits);

  __shared__ float qr[GQA][D];
  __shared__ float xd[PAGE][D + 1];  // dequantized keys, then values, of the current chunk
  __shared__ float pr[GQA][PAGE];    // probabilities of the current chunk
  __shared__ float alpha_s[GQA];
  __shared__ uint8_t valid[PAGE];

  rotate_queries<GQA>(a, sq, kvh, qr, tid);

  // running state: wave w owns heads w, w+4, ...; thread owns (head, channel) accumulators
  constexpr int HPW = (GQA + 3) / 4;       // heads per wave for the softmax
  float m_run[HPW], l_run[HPW];
#pragma unroll
  for (int i = 0; i < HPW; ++i) { m_run[i] = -INFINITY; l_run[i] = 0.0f; }
  constexpr int APT = (GQA * D + 255) / 256;  // accumulators per thread
  float acc[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) acc[i] = 0.0f;

  int n_chunks, first;
  if (bf16_split) { n_chunks = RING / PAGE; first = 0; }
  else { first = split * a.pages_per_split; n_chunks = min(a.pages_per_split, n_pages - first); }

  const size_t ring_head = (static_cast<size_t>(sq.seq) * a.hkv + kvh) * 2 * RING * D;
  const int n_win = max(0, sq.len - SINK - sq.n_int2);
  __syncthreads();

  for (int ch = 0; ch < n_chunks; ++ch) {
    // ---- stage dequantized keys of 64 tokens
    const uint8_t* blk = nullptr;
    if (!bf16_split) {
      const int lp = first + ch;
      const int page = a.page_table[static_cast<size_t>(sq.seq) * a.max_pages + lp];
      blk = a.pool + (static_cast<size_t>(page) * a.hkv + kvh) * HEAD_BLOCK;
    }
    stage_chunk(a, sq, blk, ring_head, ch, n_win, first, bf16_split, false, xd, valid, tid);
    __syncthreads();

    // ---- scores and softmax update: wave w, lane j, heads w + 4 i
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int h = wv + 4 * i;
      if (h < GQA) {
        float s = 0.0f;
        for (int c = 0; c < D; ++c) s = fmaf(qr[h][c], xd[lane][c], s);
        s = valid[lane] ? s : -INFINITY;
        const float mx = wave_max(s);
        const float m_new = fmaxf(m_run[i], mx);
        const float p = valid[lane] ? exp2f(s - m_new) : 0.0f;
        const float alpha = (m_run[i] == -INFINITY) ? 0.0f : exp2f(m_run[i] - m_new);
        l_run[i] = l_run[i] * alpha + wave_sum(p);
        m_run[i] = m_new;
        pr[h][lane] = p;
        if (lane == 0) alpha_s[h] = alpha;
      }
    }
    __syncthreads();
    stage_chunk(a, sq, blk, ring_head, ch, n_win, first, bf16_split, true, xd, valid, tid);
    __syncthreads();

    // ---- acc[h][c] = alpha acc + sum_j p_j v_j[c]
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int idx = tid + 256 * i;
      if (idx < GQA * D) {
        const int h = idx / D, c = idx % D;
        float s = acc[i] * alpha_s[h];
        for (int j = 0; j < PAGE; ++j) s = fmaf(pr[h][j], xd[j][c], s);
        acc[i] = s;
      }
    }
    __syncthreads();
  }

  // ---- partials: [m, l, o[128]] per (seq, q head, split)
  float* part = a.part;
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const int h = wv + 4 * i;
    if (h < GQA && lane == 0) {
      float* rec = part + ((static_cast<size_t>(sl) * a.hq + kvh * GQA + h) * a.n_split_max + split) * PART_STRIDE;
      rec[0] = m_run[i];
      rec[1] = l_run[i];
    }
  }
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int idx = tid + 256 * i;
    if (idx < GQA * D) {
      const int h = idx / D, c = idx % D;
      float* rec = part + ((static_cast<size_t>(sl) * a.hq + kvh * GQA + h) * a.n_split_max + split) * PART_STRIDE;
      rec[2 + c] = acc[i];
    }
  }
}

// ------------------------------------------------------------------ combine
// Grid (q heads, sequences of this chunk), S x 128 threads (S = 1 .. 4 slices, enough for the
// call's records in one pass where possible): out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i
// over the unit's records i.  Thread (slice, c) takes channel c of the records 16 slice + 16 S k
// + j (j < 16) with a running maximum of its own, so that all 16 records' loads of a pass are
// issued at once and nothing waits for a maximum over the whole unit; the slices are then
// merged.  The weights use the hardware exp2 (arguments <= 0; results below 2^-126 flush to 0).

constexpr int COMBINE_SLICES = 4, COMBINE_BATCH = 16;

__global__ __launch_bounds__(COMBINE_SLICES * D) void k_combine(DecodeArgs a) {
  // a slice is two whole waves: its index is wave-uniform
  const int h = blockIdx.x, sl = blockIdx.y, c = threadIdx.x & (D - 1);
  const int slice = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 7));
  const int n_slices = blockDim.x >> 7;
  const DecodeSeq sq = a.seqs[sl];
  const int n = unit_records(sq.n_int2, sq.len, a.pages_per_split, a.kernel);
  const float* rec0 = a.part + (static_cast<size_t>(sl) * a.hq + h) * a.n_split_max * PART_STRIDE;
  // (m, l) of a record are wave-uniform: read through the scalar cache (the records were written
  // by an earlier launch), leaving the vector loads to the channel values
  const __attribute__((address_space(4))) float* rec0_s = (const __attribute__((address_space(4))) float*)(rec0);
  float M = -INFINITY, L = 0.0f, O = 0.0f;
  for (int b = COMBINE_BATCH * slice; b < n; b += n_slices * COMBINE_BATCH) {
    float m[COMBINE_BATCH], l[COMBINE_BATCH], o[COMBINE_BATCH];
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j) {
      const size_t r = static_cast<size_t>(min(b + j, n - 1)) * PART_STRIDE;  // in range
      m[j] = rec0_s[r];
      l[j] = rec0_s[r + 1];
      o[j] = rec0[r + 2 + c];
    }
    float mb = M;
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j)
      if (b + j < n) mb = fmaxf(mb, m[j]);
    if (mb == -INFINITY) continue;  // only empty records so far (m = -inf, l = 0, o = 0)
    const float alpha = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - mb);
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j) {
      const float w = (b + j < n && m[j] != -INFINITY) ? __builtin_amdgcn_exp2f(m[j] - mb) : 0.0f;
      L = fmaf(w, l[j], L);
      O = fmaf(w, o[j], O);
    }
    M = mb;
  }
  __shared__ float sm[COMBINE_SLICES], sls[COMBINE_SLICES], so[COMBINE_SLICES][D];
  if (c == 0) {
    sm[slice] = M;
    sls[slice] = L;
  }
  so[slice][c] = O;
  __syncthreads();
  if (slice != 0) return;
  float Mt = sm[0];
  for (int p = 1; p < n_slices; ++p) Mt = fmaxf(Mt, sm[p]);
  float Lt = 0.0f, Ot = 0.0f;
  for (int p = 0; p < n_slices; ++p) {
    const float w = (sm[p] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(sm[p] - Mt);
    Lt = fmaf(w, sls[p], Lt);
    Ot = fmaf(w, so[p][c], Ot);
  }
  const size_t o = (static_cast<size_t>(sq.src) * a.hq + h) * D + c;
  if (a.out_bf16) reinterpret_cast<uint16_t*>(a.out)[o] = f32_to_bf16(Ot / Lt);
  else a.out[o] = Ot / Lt;
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t s) {
  const int slices = std::min(COMBINE_SLICES, std::max(1, (a.n_split_max + COMBINE_BATCH - 1) / COMBINE_BATCH));
  hipLaunchKernelGGL(k_combine, dim3(a.hq, a.n_seqs), dim3(slices * D), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_simple(const DecodeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  const dim3 grid(a.n_split_max, a.hkv, a.n_seqs);
  const int gqa = a.hq / a.hkv;
  if (t0) {
    const hipError_t e = hipEventRecord(t0, s);
    if (e != hipSuccess) return e;
  }
  switch (gqa) {
    case 1: hipLaunchKernelGGL(k_decode_simple<1>, grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_decode_simple<2>, grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_decode_simple<4>, grid, dim3(256), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_decode_simple<8>, grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  if (t1) {
    const hipError_t e = hipEventRecord(t1, s);
    if (e != hipSuccess) return e;
  }
  return hipGetLastError();
}

}  // namespace oscar
