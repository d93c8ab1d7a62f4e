// Internal launch interface between the host runtime (oscar_host.cpp) and the
// HIP kernels.  Per-call plans travel in kernel arguments (at most CHUNK
// sequences per launch), so a decode step needs no host-to-device copies.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oscar {

constexpr int CHUNK = 64;          // sequences per launch
constexpr int SCATTER_MAX = 224;   // page-table updates per scatter launch

// A run of consecutive page-table entries (one sequence's new pages) in one launch.
constexpr int RUN_MAX = 1000;
struct RunArgs {
  int32_t* dst;   // first entry of the run
  int32_t n;
  int32_t val[RUN_MAX];
};

struct ScatterArgs {
  int32_t* dst;
  int32_t n;
  int32_t idx[SCATTER_MAX];
  int32_t val[SCATTER_MAX];
};

struct WriteSeq {
  int32_t seq;   // sequence slot
  int32_t len0;  // length before the call
  int32_t src;   // row of this sequence in the call's k/v arrays
  int32_t pad;
};

struct WriteArgs {
  const uint16_t* k;  // bf16 [n_seqs_call][n_new][hkv][128]
  const uint16_t* v;
  uint8_t* pool;
  uint16_t* ring;
  const int32_t* page_table;
  const uint8_t* rot;
  int32_t hkv, max_pages, n_new, n_seqs;
  int32_t tiles_per_wg;  // k_write: 64-position tiles per work-group (set by launch_write)
  WriteSeq seqs[CHUNK];
};

struct EvictSeq {
  int32_t seq;
  int32_t n_int2;  // INT2 count before the call
};

// The decode step's write: per sequence, evict the oldest window token when the window is full,
// then append one token.
struct StepSeq {
  int32_t seq;
  int32_t len0;    // length before the call
  int32_t n_int2;  // INT2 count before the call
  int32_t src;     // row of this sequence in the call's k/v arrays
  int32_t evict;   // 1: the window is full, evict its oldest token first
  int32_t page;    // with evict: physical page of INT2 index n_int2 (the evicted token's page)
};

struct StepArgs {
  const uint16_t* k;  // bf16 [n_seqs_call][hkv][128]
  const uint16_t* v;
  uint8_t* pool;
  uint16_t* ring;
  const int32_t* page_table;
  const uint8_t* rot;
  int32_t hkv, max_pages, n_seqs;
  StepSeq seqs[CHUNK];
};

struct EvictArgs {
  uint8_t* pool;
  uint16_t* ring;
  const int32_t* page_table;
  int32_t hkv, max_pages, n_evict, n_seqs;
  EvictSeq seqs[CHUNK];
};

struct DecodeSeq {
  int32_t seq;     // sequence slot
  int32_t len;     // tokens stored
  int32_t n_int2;  // INT2 tokens
  int32_t src;     // row of this sequence in the call's q / out arrays
};

struct DecodeArgs {
  const uint16_t* q;      // bf16 [n_seqs_call][hq][128]
  const uint8_t* pool;
  const uint16_t* ring;
  const int32_t* page_table;
  const uint8_t* rot;
  float* part;            // [n_seqs][hq][n_split_max][130]: m, l, o[128]
  float* out;             // fp32 [n_seqs_call][hq][128]
  int32_t hkv, hq, max_pages, n_seqs;
  int32_t pages_per_split, n_split_max;
  float scale_log2;       // sm_scale * log2(e)
  int32_t kernel;         // 0 matrix-core split kernel, 1 reference kernel (record layout)
  int32_t share;          // matrix-core kernel: 1 = splits of a unit share their pages, 0 = fixed ranges
  int32_t out_bf16;       // 1: out holds bf16 (round to nearest even) instead of fp32
  int32_t wg_rows;        // matrix-core kernel: grid rows (the work-groups of the largest unit)
  DecodeSeq seqs[CHUNK];
};

constexpr int PART_STRIDE = 130;

// Work split of one (sequence, KV head) unit.  INT2 split s covers pages
// [s pps, min((s+1) pps, n_pages)) and writes partial record s.  The BF16 sink + window tokens
// (five 64-slot chunks of the ring) follow as records n_is .. n_is + nb - 1, where n_is is the
// number of INT2 splits: a BF16 token moves 512 bytes (key and value rows), an INT2 page 5120,
// so ten BF16 tokens weigh one page, and the BF16 work is cut into nb = ceil(weight / pps)
// (1..5) work-groups of whole chunks so that none of them outweighs an INT2 split.  On the
// matrix-core path (kernel 0) a single BF16 work-group is folded into the INT2 work when the
// last split's spare capacity (splits x pages-per-split - pages) holds its weight; that kernel
// shares pages between the splits of a unit and gives the folded work to split 0.  The
// reference kernel (kernel 1) keeps one BF16 work-group.
constexpr int RING_CHUNKS = 5;
__host__ __device__ inline int bf16_page_weight(int n_bf16) { return (n_bf16 + 9) / 10; }
__host__ __device__ inline int int2_splits(int n_int2, int pps) { return ((n_int2 + 63) / 64 + pps - 1) / pps; }
__host__ __device__ inline int bf16_splits(int n_int2, int len, int pps, int kernel) {
  if (kernel != 0) return 1;
  const int nb = (bf16_page_weight(len - n_int2) + pps - 1) / pps;
  return nb < 1 ? 1 : (nb > RING_CHUNKS ? RING_CHUNKS : nb);
}
__host__ __device__ inline bool bf16_folded(int n_int2, int len, int pps, int kernel) {
  const int n_pages = (n_int2 + 63) / 64, n_is = (n_pages + pps - 1) / pps;
  return kernel == 0 && n_is > 0 && bf16_splits(n_int2, len, pps, kernel) == 1 &&
         n_is * pps - n_pages >= bf16_page_weight(len - n_int2);
}
// partial records of one unit (the combine's count; the workspace holds the maximum per call)
__host__ __device__ inline int unit_records(int n_int2, int len, int pps, int kernel) {
  return int2_splits(n_int2, pps) + bf16_splits(n_int2, len, pps, kernel);
}
// work-groups of the split kernel for one unit
__host__ __device__ inline int unit_workgroups(int n_int2, int len, int pps, int kernel) {
  return int2_splits(n_int2, pps) + (bf16_folded(n_int2, len, pps, kernel) ? 0 : bf16_splits(n_int2, len, pps, kernel));
}

hipError_t launch_fill_i32(int32_t* dst, int64_t n, int32_t value, hipStream_t s);
hipError_t launch_scatter(const ScatterArgs& a, hipStream_t s);
hipError_t launch_run(const RunArgs& a, hipStream_t s);
hipError_t launch_write(const WriteArgs& a, int n_tiles, hipStream_t s);
hipError_t launch_append(const WriteArgs& a, hipStream_t s);   // no INT2 tokens in the call
hipError_t launch_evict(const EvictArgs& a, hipStream_t s);
hipError_t launch_step_write(const StepArgs& a, hipStream_t s);
// decode attention: prepared-query + split kernels (matrix-core path) or the reference-grade
// fp32 kernel, then the split combine
// (t0, t1: optional events recorded on s right before and after the split kernel)
// w (may be null): the decode step's write of the same sequences, run in the query preparation's
// launch (k_step_qprep) instead of a launch of its own
hipError_t launch_decode_mfma(const StepArgs* w, const DecodeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_decode_simple(const DecodeArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1);
hipError_t launch_combine(const DecodeArgs& a, hipStream_t s);
// work-groups of the decode split kernel to plan per residency round on the current device
int decode_resident_workgroups(int gqa, int kernel);

// Address of the allocation-free decode step's scratch array on the current device (looked up once
// per device with hipGetSymbolAddress, then cached); OSCAR_NOALLOC_SCRATCH_BYTES bytes.
hipError_t scratch_on_current_device(void** ptr);

// bytes of the prepared-query area that follows the split partials in the workspace,
// per (sequence of a launch chunk, KV head)
constexpr int QPREP_STRIDE = 8448;

// Workspace of one decode launch: the partial records [n_seqs][hq][n_split_max][130], the
// prepared queries [n_seqs][hkv][QPREP_STRIDE bytes], then one int32 page counter per (unit,
// record) slot.
__host__ __device__ inline size_t qprep_offset(const DecodeArgs& a) {
  return static_cast<size_t>(a.n_seqs) * a.hq * a.n_split_max * PART_STRIDE * sizeof(float);
}
__host__ __device__ inline size_t counter_offset(const DecodeArgs& a) {
  return qprep_offset(a) + static_cast<size_t>(a.n_seqs) * a.hkv * QPREP_STRIDE;
}

}  // namespace oscar
