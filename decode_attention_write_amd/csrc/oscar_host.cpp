// Host runtime of liboscar: the store handle, argument validation, the FIFO
// page allocator with its page-table mirror, split planning and the C ABI.
//
// Every call validates completely before it changes anything, so a call that
// fails validation leaves the store as it was.  A HIP failure after a call has
// committed its host bookkeeping marks the handle unusable (its mirror may be
// ahead of the device), and later calls on it are refused.  All per-call plans travel to the kernels in
// kernel arguments; the only host-to-device traffic besides that is the
// rotation upload and page-table updates (small scatter launches).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <numeric>
#include <string>
#include <vector>

#include "oscar.h"
#include "launch.h"

namespace oscar {

thread_local std::string g_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
}

}  // namespace oscar

using namespace oscar;

struct oscar_kv {
  oscar_kv_desc desc;
  bool plan_only;
  std::vector<int64_t> len;
  std::vector<int64_t> n_int2;
  std::vector<int32_t> table;  // host mirror [max_seqs][max_pages]
  std::deque<int32_t> fifo;
  int32_t pages_per_split = 0;
  int32_t decode_kernel = 0;   // 0: matrix-core kernel, 1: reference-grade fp32 kernel
  int32_t deterministic = 0;   // 1: fixed page range per split (no sharing between splits)
  int32_t write_evicts = 0;    // 1: a write that overflows a non-empty window evicts as it goes
  int32_t out_bf16 = 0;        // 1: decode outputs are written as bf16
  bool has_rotation = false;
  std::vector<float> rot_host;  // [hkv][128][128], kept for re-deriving the key-mean shift
  std::vector<float> key_mean;  // [hkv][128], empty: no key mean
  // A HIP failure after a call has committed its host bookkeeping (page table mirror, FIFO,
  // lengths) leaves the mirror ahead of the device: the handle then refuses every further call.
  bool broken = false;
  // timing events per timed kernel: 2 * OSCAR_TIMING_PAIRS each when timing is on
  std::vector<hipEvent_t> timing_ev[2];
  mutable int32_t timing_used[2] = {0, 0};  // pairs recorded since the last read (decode takes a const handle)
  ~oscar_kv() {
    for (auto& v : timing_ev)
      for (hipEvent_t e : v) (void)hipEventDestroy(e);
  }
  // next free event pair of a timed kernel, or {null, null}
  std::pair<hipEvent_t, hipEvent_t> take_timing_pair(int kind) const {
    if (timing_ev[kind].empty() || timing_used[kind] >= OSCAR_TIMING_PAIRS) return {nullptr, nullptr};
    const int i = timing_used[kind]++;
    return {timing_ev[kind][2 * i], timing_ev[kind][2 * i + 1]};
  }
};

namespace {

constexpr int64_t kSink = OSCAR_SINK_TOKENS, kWin = OSCAR_WINDOW_TOKENS, kRing = OSCAR_RING_SLOTS;
constexpr int64_t kPage = OSCAR_PAGE_TOKENS;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// bfloat16 from/to binary32 on the host: round to nearest even (finite inputs), and exact widening.
uint16_t f32_to_bf16_rn(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

float bf16_to_f32(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

int hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return OSCAR_E_HIP;
}

// A HIP failure of a call that has already moved the host mirror: mark the handle unusable.
int hip_fail_committed(oscar_kv* kv, hipError_t e, const char* what) {
  kv->broken = true;
  return hip_fail(e, what);
}

// Every call on a handle first checks that no earlier call left it unusable.
int check_usable(const oscar_kv* kv, const char* who) {
  if (!kv) { set_error("%s: null handle", who); return OSCAR_E_ARG; }
  if (kv->broken) {
    set_error("%s: the handle is unusable after a HIP failure (destroy it and create a new store)", who);
    return OSCAR_E_STATE;
  }
  return OSCAR_OK;
}

int check_desc(const oscar_kv_desc* d) {
  if (!d) { set_error("null descriptor"); return OSCAR_E_ARG; }
  if (d->num_kv_heads < 1 || d->num_q_heads < d->num_kv_heads || d->num_q_heads % d->num_kv_heads) {
    set_error("num_q_heads must be a positive multiple of num_kv_heads");
    return OSCAR_E_ARG;
  }
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) { set_error("Hq/Hkv must be 1, 2, 4 or 8"); return OSCAR_E_ARG; }
  if (d->max_seqs < 1 || d->max_pages_per_seq < 1 || d->num_pages < 1) {
    set_error("max_seqs, max_pages_per_seq and num_pages must be >= 1");
    return OSCAR_E_ARG;
  }
  if (d->flags & ~OSCAR_FLAG_PLAN_ONLY) { set_error("unknown flag bits"); return OSCAR_E_ARG; }
  return OSCAR_OK;
}

// seq ids in range and distinct
int check_seqs(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs) {
  if (!seq_ids || n_seqs < 1 || n_seqs > kv->desc.max_seqs) {
    set_error("seq_ids must hold 1..max_seqs entries");
    return OSCAR_E_ARG;
  }
  std::vector<char> seen(kv->desc.max_seqs, 0);
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    if (s < 0 || s >= kv->desc.max_seqs) { set_error("seq id %d out of range", s); return OSCAR_E_ARG; }
    if (seen[s]) { set_error("seq id %d listed twice", s); return OSCAR_E_ARG; }
    seen[s] = 1;
  }
  return OSCAR_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Push page-table updates to the device: runs of at least 64 consecutive entries (a long write
// into one sequence) go in run launches of up to RUN_MAX values, the rest in scatter launches.
int push_table(oscar_kv* kv, const std::vector<std::pair<int32_t, int32_t>>& upd, hipStream_t st) {
  if (kv->plan_only || upd.empty()) return OSCAR_OK;
  std::vector<std::pair<int32_t, int32_t>> rest;
  for (size_t i = 0; i < upd.size();) {
    size_t j = i + 1;
    while (j < upd.size() && upd[j].first == upd[j - 1].first + 1) ++j;
    if (j - i >= 64) {
      for (size_t r = i; r < j; r += RUN_MAX) {
        RunArgs a{};
        a.dst = kv->desc.page_table + upd[r].first;
        a.n = static_cast<int32_t>(std::min<size_t>(RUN_MAX, j - r));
        for (int k = 0; k < a.n; ++k) a.val[k] = upd[r + k].second;
        hipError_t e = launch_run(a, st);
        if (e != hipSuccess) return hip_fail_committed(kv, e, "page-table update");
      }
    } else {
      rest.insert(rest.end(), upd.begin() + i, upd.begin() + j);
    }
    i = j;
  }
  for (size_t i = 0; i < rest.size(); i += SCATTER_MAX) {
    ScatterArgs a{};
    a.dst = kv->desc.page_table;
    a.n = static_cast<int32_t>(std::min<size_t>(SCATTER_MAX, rest.size() - i));
    for (int k = 0; k < a.n; ++k) {
      a.idx[k] = rest[i + k].first;
      a.val[k] = rest[i + k].second;
    }
    hipError_t e = launch_scatter(a, st);
    if (e != hipSuccess) return hip_fail_committed(kv, e, "page-table update");
  }
  return OSCAR_OK;
}

// (length, INT2 count) of each listed sequence, in list order: the state a decode call plans for
struct SeqState {
  int64_t len, n2;
};

std::vector<SeqState> current_state(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs) {
  std::vector<SeqState> st(n_seqs);
  for (int i = 0; i < n_seqs; ++i) st[i] = SeqState{kv->len[seq_ids[i]], kv->n_int2[seq_ids[i]]};
  return st;
}

// The state after a decode-step write: one more token per sequence, and one more INT2 token
// where the window is full.
std::vector<SeqState> state_after_step(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs) {
  std::vector<SeqState> st = current_state(kv, seq_ids, n_seqs);
  for (SeqState& q : st) {
    if (q.len > 0 && std::max<int64_t>(0, q.len - kSink - q.n2) == kWin) q.n2 += 1;
    q.len += 1;
  }
  return st;
}

int64_t choose_pages_per_split(const oscar_kv* kv, int32_t n_seqs, const std::vector<SeqState>& st) {
  if (kv->pages_per_split > 0) return kv->pages_per_split;
  // Work-groups of the split kernel that fit on the device at once (the matrix-core kernel uses
  // one wavefront per work-group).  Aim for a single residency round holding as many waves as
  // fit: the smallest pages-per-split whose work-groups (INT2 splits, plus a sink/window
  // work-group where it is not folded into the last INT2 split) fit the resident capacity, for
  // each launch chunk of up to CHUNK sequences.
  if (kv->plan_only) return 64;
  const int64_t resident = decode_resident_workgroups(kv->desc.num_q_heads / kv->desc.num_kv_heads,
                                                      kv->decode_kernel);
  const int64_t hkv = kv->desc.num_kv_heads;
  int64_t best = 1;
  for (int c0 = 0; c0 < n_seqs; c0 += CHUNK) {
    const int n = std::min(CHUNK, n_seqs - c0);
    int64_t max_pages = 0, total = 0;
    for (int i = c0; i < c0 + n; ++i) {
      const int64_t p = ceil_div(st[i].n2, kPage);
      max_pages = std::max(max_pages, p);
      total += p;
    }
    if (max_pages == 0) continue;
    const int kernel = kv->decode_kernel;
    auto wgs_for = [&](int64_t pps) {
      int64_t w = 0;
      for (int i = c0; i < c0 + n; ++i)
        w += unit_workgroups(static_cast<int>(st[i].n2), static_cast<int>(st[i].len), static_cast<int>(pps), kernel);
      return w * hkv;
    };
    const int64_t budget = std::max<int64_t>(n * hkv, resident);
    int64_t pps = std::max<int64_t>(1, ceil_div(total * hkv, budget));
    for (; pps < max_pages; ++pps)
      if (wgs_for(pps) <= budget) break;
    best = std::max(best, pps);
  }
  // Fixed page ranges (the deterministic mode) cannot move work between the splits of a unit:
  // with two residency rounds of half the size, the dispatcher gives the second round to the
  // slots that finish first.  Measured on the 100000 x 32 layer (142 pages per split in one
  // round): split kernel 404-410 us against 376-380 us at 71; no gain where a split holds
  // fewer pages (8 x 32768 at 13 -> 7 or 9, ragged GQA-8 at 87 -> 44).
  if (kv->deterministic && kv->decode_kernel == 0 && best >= 100) best = ceil_div(best, 2);
  return best;
}

// The launch plan of one chunk of sequences [c0, c0 + n) of st: record slots per unit, grid rows
// of the split kernel, and the launch order of the sequences.  A sequence's INT2 work-groups each
// hold about full pages / INT2 splits pages, and its units end in the order of that load (16
// sequences of U[8192, 131072] tokens, GQA 8: between 140 and 195 us); the sequences go into the
// launch most loaded first (stable), so that their work-groups are dispatched first in every grid
// row.  Split kernel on that layer: 196-198 -> 192-194 us (interleaved runs).
struct ChunkPlan {
  std::vector<int> order;   // chunk positions in launch order
  int64_t records = 1;      // record slots per unit
  int64_t wg_rows = 1;      // grid rows of the split kernel
};

ChunkPlan plan_chunk(const oscar_kv* kv, const std::vector<SeqState>& st, int c0, int n, int64_t pps) {
  ChunkPlan p;
  p.order.resize(n);
  std::iota(p.order.begin(), p.order.end(), 0);
  const int kernel = kv->decode_kernel;
  std::vector<double> load(n, 0.0);
  for (int i = 0; i < n; ++i) {
    const int n2 = static_cast<int>(st[c0 + i].n2), len = static_cast<int>(st[c0 + i].len);
    p.records = std::max<int64_t>(p.records, unit_records(n2, len, static_cast<int>(pps), kernel));
    p.wg_rows = std::max<int64_t>(p.wg_rows, unit_workgroups(n2, len, static_cast<int>(pps), kernel));
    const int full = n2 / static_cast<int>(kPage);
    if (full > 0) load[i] = static_cast<double>(full) / int2_splits(n2, static_cast<int>(pps));
  }
  std::stable_sort(p.order.begin(), p.order.end(), [&](int x, int y) { return load[x] > load[y]; });
  return p;
}

// Evictions a write of n_new tokens into the non-empty sequence s needs: the sink and window
// hold 320 - (len - n_int2) more tokens; every token beyond that first moves the oldest window
// token into INT2.
int64_t overflow_evictions(const oscar_kv* kv, int s, int64_t n_new) {
  return std::max<int64_t>(0, n_new - (kRing - (kv->len[s] - kv->n_int2[s])));
}

// Workspace bytes of a decode call over sequences in state st: split partials, then the prepared
// queries, then one page counter per record slot (matrix-core kernel); sized for the largest chunk.
size_t workspace_bytes_for(const oscar_kv* kv, int32_t n_seqs, const std::vector<SeqState>& st) {
  const int64_t pps = choose_pages_per_split(kv, n_seqs, st);
  int64_t max_split = 1;
  for (int c0 = 0; c0 < n_seqs; c0 += CHUNK)
    max_split = std::max(max_split, plan_chunk(kv, st, c0, std::min(CHUNK, n_seqs - c0), pps).records);
  const int64_t rows = std::min<int64_t>(n_seqs, CHUNK);
  return static_cast<size_t>(rows) * kv->desc.num_q_heads * max_split * PART_STRIDE * sizeof(float) +
         static_cast<size_t>(rows) * kv->desc.num_kv_heads * QPREP_STRIDE +
         static_cast<size_t>(rows) * kv->desc.num_kv_heads * max_split * sizeof(int32_t);
}

// ---- decode-step write and decode attention, shared by the one-call and two-call forms

// Validation of a decode-step write (nothing is changed).
int check_step_write(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const void* k, const void* v,
                     const char* who) {
  int rc = check_usable(kv, who);
  if (rc) return rc;
  rc = check_seqs(kv, seq_ids, n_seqs);
  if (rc) return rc;
  if (!kv->plan_only && (!k || !v)) { set_error("%s: null k or v", who); return OSCAR_E_ARG; }
  if (!kv->has_rotation) { set_error("%s: rotation not set", who); return OSCAR_E_STATE; }
  const int64_t maxp = kv->desc.max_pages_per_seq;
  int64_t need = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    if (kv->len[s] == 0) {
      set_error("%s: sequence %d is empty (its first write takes oscar_kv_write)", who, s);
      return OSCAR_E_STATE;
    }
    const int64_t win = std::max<int64_t>(0, kv->len[s] - kSink - kv->n_int2[s]);
    if (win == kWin && kv->n_int2[s] % kPage == 0) {
      if (kv->n_int2[s] / kPage + 1 > maxp) {
        set_error("%s: sequence %d exceeds max_pages_per_seq", who, s);
        return OSCAR_E_NOPAGE;
      }
      ++need;
    }
  }
  if (need > static_cast<int64_t>(kv->fifo.size())) {
    set_error("%s: needs %lld pages, %zu free", who, static_cast<long long>(need), kv->fifo.size());
    return OSCAR_E_NOPAGE;
  }
  return OSCAR_OK;
}

// Host state of a validated decode-step write: evict where the window is full (a page from the
// FIFO when the INT2 index is a multiple of 64), then one more token per sequence.
std::vector<StepSeq> commit_step_write(oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs,
                                       std::vector<std::pair<int32_t, int32_t>>& upd) {
  const int64_t maxp = kv->desc.max_pages_per_seq;
  std::vector<StepSeq> plan(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    const int64_t win = std::max<int64_t>(0, kv->len[s] - kSink - kv->n_int2[s]);
    const bool ev = (win == kWin);
    plan[i] = StepSeq{s, static_cast<int32_t>(kv->len[s]), static_cast<int32_t>(kv->n_int2[s]), i, ev ? 1 : 0, -1};
    if (ev) {
      const int32_t idx = static_cast<int32_t>(s * maxp + kv->n_int2[s] / kPage);
      if (kv->n_int2[s] % kPage == 0) {
        const int32_t page = kv->fifo.front();
        kv->fifo.pop_front();
        kv->table[idx] = page;
        upd.emplace_back(idx, page);
      }
      plan[i].page = kv->table[idx];
      kv->n_int2[s] += 1;
    }
    kv->len[s] += 1;
  }
  return plan;
}

StepArgs step_args(const oscar_kv* kv, const void* k, const void* v, const std::vector<StepSeq>& plan, int c0, int n) {
  StepArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.pool = static_cast<uint8_t*>(kv->desc.pool);
  a.ring = static_cast<uint16_t*>(kv->desc.ring);
  a.page_table = kv->desc.page_table;
  a.rot = static_cast<const uint8_t*>(kv->desc.rot);
  a.hkv = kv->desc.num_kv_heads;
  a.max_pages = kv->desc.max_pages_per_seq;
  a.n_seqs = n;
  for (int i = 0; i < n; ++i) a.seqs[i] = plan[c0 + i];
  return a;
}

// Validation of a decode-attention call apart from its workspace size (nothing is changed).
int check_decode(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const void* q, float sm_scale,
                 const float* out, const void* ws, const char* who) {
  int rc = check_usable(kv, who);
  if (rc) return rc;
  rc = check_seqs(kv, seq_ids, n_seqs);
  if (rc) return rc;
  if (!kv->plan_only && (!q || !out || !ws)) { set_error("%s: null q, out or workspace", who); return OSCAR_E_ARG; }
  if (!std::isfinite(sm_scale)) { set_error("%s: non-finite sm_scale", who); return OSCAR_E_ARG; }
  if (!kv->has_rotation) { set_error("%s: rotation not set", who); return OSCAR_E_STATE; }
  for (int i = 0; i < n_seqs; ++i)
    if (kv->len[seq_ids[i]] == 0) { set_error("%s: sequence %d is empty", who, seq_ids[i]); return OSCAR_E_STATE; }
  return OSCAR_OK;
}

// Decode attention launches over the current host state, chunk by chunk.  With a step plan (the
// sequences' decode-step write, already committed to the host state) the write runs in the
// query preparation's launch.
int launch_decode(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const std::vector<StepSeq>* plan,
                  const void* q, float sm_scale, float* out, void* ws, hipStream_t st, const char* who,
                  const void* k = nullptr, const void* v = nullptr) {
  const std::vector<SeqState> state = current_state(kv, seq_ids, n_seqs);
  const int64_t pps = choose_pages_per_split(kv, n_seqs, state);
  for (int c0 = 0; c0 < n_seqs; c0 += CHUNK) {
    const ChunkPlan p = plan_chunk(kv, state, c0, std::min(CHUNK, n_seqs - c0), pps);
    DecodeArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.pool = static_cast<const uint8_t*>(kv->desc.pool);
    a.ring = static_cast<const uint16_t*>(kv->desc.ring);
    a.page_table = kv->desc.page_table;
    a.rot = static_cast<const uint8_t*>(kv->desc.rot);
    a.part = static_cast<float*>(ws);
    a.out = out;
    a.hkv = kv->desc.num_kv_heads;
    a.hq = kv->desc.num_q_heads;
    a.max_pages = kv->desc.max_pages_per_seq;
    a.n_seqs = std::min(CHUNK, n_seqs - c0);
    a.pages_per_split = static_cast<int32_t>(pps);
    for (int i = 0; i < a.n_seqs; ++i) {
      const int j = c0 + p.order[i];
      const int s = seq_ids[j];
      a.seqs[i] = DecodeSeq{s, static_cast<int32_t>(kv->len[s]), static_cast<int32_t>(kv->n_int2[s]), j};
    }
    a.n_split_max = static_cast<int32_t>(p.records);
    a.wg_rows = static_cast<int32_t>(p.wg_rows);
    a.kernel = kv->decode_kernel;
    a.share = kv->deterministic ? 0 : 1;
    a.out_bf16 = kv->out_bf16;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    const auto [t0, t1] = kv->take_timing_pair(OSCAR_TIMED_DECODE);
    hipError_t e;
    if (kv->decode_kernel == 1) {
      e = launch_decode_simple(a, st, t0, t1);
    } else if (plan) {
      const StepArgs w = step_args(kv, k, v, *plan, c0, a.n_seqs);
      e = launch_decode_mfma(&w, a, st, t0, t1);
    } else {
      e = launch_decode_mfma(nullptr, a, st, t0, t1);
    }
    if (e == hipSuccess) e = launch_combine(a, st);
    if (e != hipSuccess) return hip_fail(e, who);
  }
  return OSCAR_OK;
}

}  // namespace

extern "C" {

const char* oscar_last_error(void) { return g_error.c_str(); }

int oscar_kv_buffer_bytes(const oscar_kv_desc* d, size_t* pool, size_t* ring, size_t* table, size_t* rot) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (pool) *pool = static_cast<size_t>(d->num_pages) * d->num_kv_heads * OSCAR_HEAD_BLOCK;
  if (ring) *ring = static_cast<size_t>(d->max_seqs) * d->num_kv_heads * 2 * kRing * OSCAR_HEAD_DIM * 2;
  if (table) *table = static_cast<size_t>(d->max_seqs) * d->max_pages_per_seq * 4;
  if (rot) *rot = static_cast<size_t>(d->num_kv_heads) * OSCAR_ROT_HEAD_BYTES;
  return OSCAR_OK;
}

int oscar_kv_create(const oscar_kv_desc* d, const int32_t* free_pages, int32_t n_free, void* stream, oscar_kv** out) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (!out || (n_free > 0 && !free_pages) || n_free < 0 || n_free > d->num_pages) {
    set_error("oscar_kv_create: bad free list or output pointer");
    return OSCAR_E_ARG;
  }
  const bool plan = (d->flags & OSCAR_FLAG_PLAN_ONLY) != 0;
  if (!plan && (!d->pool || !d->ring || !d->page_table || !d->rot)) {
    set_error("oscar_kv_create: device buffers must be set (or OSCAR_FLAG_PLAN_ONLY)");
    return OSCAR_E_ARG;
  }
  std::vector<char> seen(d->num_pages, 0);
  for (int i = 0; i < n_free; ++i) {
    const int p = free_pages[i];
    if (p < 0 || p >= d->num_pages || seen[p]) {
      set_error("oscar_kv_create: free page %d out of range or repeated", p);
      return OSCAR_E_ARG;
    }
    seen[p] = 1;
  }
  oscar_kv* kv = new oscar_kv();
  kv->desc = *d;
  kv->plan_only = plan;
  kv->len.assign(d->max_seqs, 0);
  kv->n_int2.assign(d->max_seqs, 0);
  kv->table.assign(static_cast<size_t>(d->max_seqs) * d->max_pages_per_seq, -1);
  kv->fifo.assign(free_pages, free_pages + n_free);
  if (!plan) {
    hipError_t e = launch_fill_i32(d->page_table, static_cast<int64_t>(kv->table.size()), -1, as_stream(stream));
    if (e != hipSuccess) {
      delete kv;
      return hip_fail(e, "oscar_kv_create: page-table fill");
    }
  }
  *out = kv;
  return OSCAR_OK;
}

void oscar_kv_destroy(oscar_kv* kv) { delete kv; }

// The device rotation block of every head from the handle's host rotation and key mean: fp32 R,
// three bf16 terms r0 + r1 + r2 ~= R (r0 = bf16(R), r1 = bf16(R - r0), r2 = bf16(R - r0 - r1); the
// fp32 differences are exact, |R - r0 - r1 - r2| <= 2^-24 |R|) stored transposed ([term][output
// channel c][input channel i]) for the write kernel's MFMA A operand, then fp32 -(mu . R) (the dot
// products in fp64, rounded once; +0 where zero, so that a zero mean leaves every sum as it is).
// Uploaded on stream; returns after the copy has consumed the host buffer.
static int upload_rotation(oscar_kv* kv, void* stream, const char* who) {
  const int hkv = kv->desc.num_kv_heads;
  const size_t dd = OSCAR_HEAD_DIM * OSCAR_HEAD_DIM;
  std::vector<uint8_t> blob(static_cast<size_t>(hkv) * OSCAR_ROT_HEAD_BYTES, 0);
  for (int h = 0; h < hkv; ++h) {
    const float* rh = kv->rot_host.data() + h * dd;
    uint8_t* base = blob.data() + static_cast<size_t>(h) * OSCAR_ROT_HEAD_BYTES;
    std::memcpy(base, rh, dd * 4);
    uint16_t* terms = reinterpret_cast<uint16_t*>(base + dd * 4);
    for (size_t i = 0; i < OSCAR_HEAD_DIM; ++i)
      for (size_t c = 0; c < OSCAR_HEAD_DIM; ++c) {
        const float r = rh[i * OSCAR_HEAD_DIM + c];
        const uint16_t t0 = f32_to_bf16_rn(r);
        const float d1 = r - bf16_to_f32(t0);
        const uint16_t t1 = f32_to_bf16_rn(d1);
        const uint16_t t2 = f32_to_bf16_rn(d1 - bf16_to_f32(t1));
        terms[c * OSCAR_HEAD_DIM + i] = t0;
        terms[dd + c * OSCAR_HEAD_DIM + i] = t1;
        terms[2 * dd + c * OSCAR_HEAD_DIM + i] = t2;
      }
    float* nmu = reinterpret_cast<float*>(base + dd * 4 + 3 * dd * 2);
    for (size_t c = 0; c < OSCAR_HEAD_DIM; ++c) {
      double m = 0.0;
      if (!kv->key_mean.empty())
        for (size_t i = 0; i < OSCAR_HEAD_DIM; ++i)
          m += static_cast<double>(kv->key_mean[h * OSCAR_HEAD_DIM + i]) * static_cast<double>(rh[i * OSCAR_HEAD_DIM + c]);
      const float v = static_cast<float>(-m);
      nmu[c] = (v == 0.0f) ? 0.0f : v;
    }
  }
  hipError_t e = hipMemcpyAsync(kv->desc.rot, blob.data(), blob.size(), hipMemcpyHostToDevice, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  // the host blob dies at return: make sure the (pageable) copy has consumed it
  e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, who);
  return OSCAR_OK;
}

int oscar_kv_set_rotation(oscar_kv* kv, const float* rot_host, void* stream) {
  if (!kv || !rot_host) { set_error("oscar_kv_set_rotation: null argument"); return OSCAR_E_ARG; }
  if (int rc = check_usable(kv, "oscar_kv_set_rotation")) return rc;
  const int hkv = kv->desc.num_kv_heads;
  const size_t n = static_cast<size_t>(hkv) * OSCAR_HEAD_DIM * OSCAR_HEAD_DIM;
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(rot_host[i])) { set_error("oscar_kv_set_rotation: non-finite entry"); return OSCAR_E_NUMERIC; }
  kv->rot_host.assign(rot_host, rot_host + n);
  if (!kv->plan_only)
    if (int rc = upload_rotation(kv, stream, "oscar_kv_set_rotation: upload")) return rc;
  kv->has_rotation = true;
  return OSCAR_OK;
}

int oscar_kv_set_key_mean(oscar_kv* kv, const float* mean, void* stream) {
  if (!kv) { set_error("oscar_kv_set_key_mean: null handle"); return OSCAR_E_ARG; }
  if (int rc = check_usable(kv, "oscar_kv_set_key_mean")) return rc;
  const size_t n = static_cast<size_t>(kv->desc.num_kv_heads) * OSCAR_HEAD_DIM;
  if (mean) {
    for (size_t i = 0; i < n; ++i)
      if (!std::isfinite(mean[i])) { set_error("oscar_kv_set_key_mean: non-finite entry"); return OSCAR_E_ARG; }
    kv->key_mean.assign(mean, mean + n);
  } else {
    kv->key_mean.clear();
  }
  if (kv->has_rotation && !kv->plan_only)
    return upload_rotation(kv, stream, "oscar_kv_set_key_mean: upload");
  return OSCAR_OK;
}

int oscar_kv_write(oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, int32_t n_new, const void* k,
                   const void* v, void* stream) {
  int rc = check_usable(kv, "oscar_kv_write");
  if (rc) return rc;
  rc = check_seqs(kv, seq_ids, n_seqs);
  if (rc) return rc;
  if (n_new < 1) { set_error("oscar_kv_write: n_new must be >= 1"); return OSCAR_E_ARG; }
  if (!kv->plan_only && (!k || !v)) { set_error("oscar_kv_write: null k or v"); return OSCAR_E_ARG; }
  if (!kv->has_rotation) { set_error("oscar_kv_write: rotation not set"); return OSCAR_E_STATE; }
  const int64_t maxp = kv->desc.max_pages_per_seq;
  int64_t need = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    if (kv->len[s] == 0) {
      const int64_t pages = ceil_div(std::max<int64_t>(0, n_new - kRing), kPage);
      if (pages > maxp) {
        set_error("oscar_kv_write: sequence %d would need %lld pages > max_pages_per_seq", s, static_cast<long long>(pages));
        return OSCAR_E_NOPAGE;
      }
      need += pages;
    } else {
      const int64_t e = overflow_evictions(kv, s, n_new);
      if (e > 0 && !kv->write_evicts) {
        set_error("oscar_kv_write: window of sequence %d would hold %lld > 256 tokens", s,
                  static_cast<long long>(kWin + e));
        return OSCAR_E_WINDOW_FULL;
      }
      const int64_t n2 = kv->n_int2[s];
      if (ceil_div(n2 + e, kPage) > maxp) {
        set_error("oscar_kv_write: sequence %d would need %lld pages > max_pages_per_seq", s,
                  static_cast<long long>(ceil_div(n2 + e, kPage)));
        return OSCAR_E_NOPAGE;
      }
      need += ceil_div(n2 + e, kPage) - ceil_div(n2, kPage);
    }
  }
  if (need > static_cast<int64_t>(kv->fifo.size())) {
    set_error("oscar_kv_write: needs %lld pages, %zu free", static_cast<long long>(need), kv->fifo.size());
    return OSCAR_E_NOPAGE;
  }
  // ---- commit: allocate pages, update mirrors
  std::vector<std::pair<int32_t, int32_t>> upd;
  std::vector<WriteSeq> plan, over;   // plain writes; writes that evict as they go
  std::vector<int64_t> over_n2;       // INT2 count before the call, per evicting write
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    const int64_t e = (kv->len[s] == 0) ? 0 : overflow_evictions(kv, s, n_new);
    if (e > 0) {
      over.push_back(WriteSeq{s, static_cast<int32_t>(kv->len[s]), i, 0});
      over_n2.push_back(kv->n_int2[s]);
      for (int64_t p = ceil_div(kv->n_int2[s], kPage); p < ceil_div(kv->n_int2[s] + e, kPage); ++p) {
        const int32_t page = kv->fifo.front();
        kv->fifo.pop_front();
        const int32_t idx = static_cast<int32_t>(s * maxp + p);
        kv->table[idx] = page;
        upd.emplace_back(idx, page);
      }
      kv->n_int2[s] += e;
      kv->len[s] += n_new;
      continue;
    }
    plan.push_back(WriteSeq{s, static_cast<int32_t>(kv->len[s]), i, 0});
    if (kv->len[s] == 0) {
      const int64_t n2 = std::max<int64_t>(0, n_new - kRing);
      for (int64_t p = 0; p < ceil_div(n2, kPage); ++p) {
        const int32_t page = kv->fifo.front();
        kv->fifo.pop_front();
        const int32_t idx = static_cast<int32_t>(s * maxp + p);
        kv->table[idx] = page;
        upd.emplace_back(idx, page);
      }
      kv->n_int2[s] = n2;
    }
    kv->len[s] += n_new;
  }
  if (kv->plan_only) return OSCAR_OK;
  hipStream_t st = as_stream(stream);
  rc = push_table(kv, upd, st);
  if (rc) return rc;
  const int n_tiles = static_cast<int>(ceil_div(n_new, kPage));
  // a call that produces no INT2 token (appends, short first writes) takes the per-token kernel
  bool any_int2 = false;
  for (const WriteSeq& w : plan) any_int2 |= (w.len0 == 0 && n_new > kRing);
  const int n_plain = static_cast<int>(plan.size());
  for (int c0 = 0; c0 < n_plain; c0 += CHUNK) {
    WriteArgs a{};
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.pool = static_cast<uint8_t*>(kv->desc.pool);
    a.ring = static_cast<uint16_t*>(kv->desc.ring);
    a.page_table = kv->desc.page_table;
    a.rot = static_cast<const uint8_t*>(kv->desc.rot);
    a.hkv = kv->desc.num_kv_heads;
    a.max_pages = kv->desc.max_pages_per_seq;
    a.n_new = n_new;
    a.n_seqs = std::min(CHUNK, n_plain - c0);
    for (int i = 0; i < a.n_seqs; ++i) a.seqs[i] = plan[c0 + i];
    const auto [t0, t1] = kv->take_timing_pair(OSCAR_TIMED_WRITE);
    hipError_t e = t0 ? hipEventRecord(t0, st) : hipSuccess;
    if (e == hipSuccess) e = any_int2 ? launch_write(a, n_tiles, st) : launch_append(a, st);
    if (e == hipSuccess && t1) e = hipEventRecord(t1, st);
    if (e != hipSuccess) return hip_fail_committed(kv, e, "oscar_kv_write: launch");
  }
  // Writes that overflow a non-empty window, one sequence at a time: the tokens that fit, then
  // rounds of (evict the c oldest window tokens, append the next c tokens), c <= 256.  The c
  // tokens of a round land in the ring slots its eviction has just read, so each round equals c
  // alternations of single-token eviction and append.
  const size_t row = static_cast<size_t>(kv->desc.num_kv_heads) * OSCAR_HEAD_DIM;
  for (size_t j = 0; j < over.size(); ++j) {
    const WriteSeq& w = over[j];
    int64_t len = w.len0, n2 = over_n2[j], t0 = 0;
    while (t0 < n_new) {
      const int64_t room = kRing - (len - n2);   // free sink + window slots
      const int64_t c = (room > 0) ? std::min<int64_t>(room, n_new - t0) : std::min<int64_t>(kWin, n_new - t0);
      hipError_t e = hipSuccess;
      if (room <= 0) {
        EvictArgs ea{};
        ea.pool = static_cast<uint8_t*>(kv->desc.pool);
        ea.ring = static_cast<uint16_t*>(kv->desc.ring);
        ea.page_table = kv->desc.page_table;
        ea.hkv = kv->desc.num_kv_heads;
        ea.max_pages = kv->desc.max_pages_per_seq;
        ea.n_evict = static_cast<int32_t>(c);
        ea.n_seqs = 1;
        ea.seqs[0] = EvictSeq{w.seq, static_cast<int32_t>(n2)};
        e = launch_evict(ea, st);
        n2 += c;
      }
      if (e == hipSuccess) {
        WriteArgs a{};
        const size_t off = (static_cast<size_t>(w.src) * n_new + t0) * row;
        a.k = static_cast<const uint16_t*>(k) + off;
        a.v = static_cast<const uint16_t*>(v) + off;
        a.pool = static_cast<uint8_t*>(kv->desc.pool);
        a.ring = static_cast<uint16_t*>(kv->desc.ring);
        a.page_table = kv->desc.page_table;
        a.rot = static_cast<const uint8_t*>(kv->desc.rot);
        a.hkv = kv->desc.num_kv_heads;
        a.max_pages = kv->desc.max_pages_per_seq;
        a.n_new = static_cast<int32_t>(c);
        a.n_seqs = 1;
        a.seqs[0] = WriteSeq{w.seq, static_cast<int32_t>(len), 0, 0};
        e = launch_append(a, st);
      }
      if (e != hipSuccess) return hip_fail_committed(kv, e, "oscar_kv_write: launch");
      len += c;
      t0 += c;
    }
  }
  return OSCAR_OK;
}

int oscar_kv_set_output_bf16(oscar_kv* kv, int32_t on) {
  if (!kv || (on != 0 && on != 1)) { set_error("oscar_kv_set_output_bf16: bad handle or value"); return OSCAR_E_ARG; }
  kv->out_bf16 = on;
  return OSCAR_OK;
}

int oscar_kv_set_write_evicts(oscar_kv* kv, int32_t on) {
  if (!kv || (on != 0 && on != 1)) { set_error("oscar_kv_set_write_evicts: bad handle or value"); return OSCAR_E_ARG; }
  kv->write_evicts = on;
  return OSCAR_OK;
}

int oscar_kv_evict_window(oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, int32_t n_evict, void* stream) {
  int rc = check_usable(kv, "oscar_kv_evict_window");
  if (rc) return rc;
  rc = check_seqs(kv, seq_ids, n_seqs);
  if (rc) return rc;
  if (n_evict < 1) { set_error("oscar_kv_evict_window: n_evict must be >= 1"); return OSCAR_E_ARG; }
  const int64_t maxp = kv->desc.max_pages_per_seq;
  int64_t need = 0;
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    const int64_t win = std::max<int64_t>(0, kv->len[s] - kSink - kv->n_int2[s]);
    if (win < n_evict) {
      set_error("oscar_kv_evict_window: sequence %d holds %lld window tokens < %d", s, static_cast<long long>(win), n_evict);
      return OSCAR_E_WINDOW_SHORT;
    }
    const int64_t p_before = ceil_div(kv->n_int2[s], kPage), p_after = ceil_div(kv->n_int2[s] + n_evict, kPage);
    if (p_after > maxp) { set_error("oscar_kv_evict_window: sequence %d exceeds max_pages_per_seq", s); return OSCAR_E_NOPAGE; }
    need += p_after - p_before;
  }
  if (need > static_cast<int64_t>(kv->fifo.size())) {
    set_error("oscar_kv_evict_window: needs %lld pages, %zu free", static_cast<long long>(need), kv->fifo.size());
    return OSCAR_E_NOPAGE;
  }
  std::vector<std::pair<int32_t, int32_t>> upd;
  std::vector<EvictSeq> plan(n_seqs);
  for (int i = 0; i < n_seqs; ++i) {
    const int s = seq_ids[i];
    plan[i] = EvictSeq{s, static_cast<int32_t>(kv->n_int2[s])};
    const int64_t p_before = ceil_div(kv->n_int2[s], kPage), p_after = ceil_div(kv->n_int2[s] + n_evict, kPage);
    for (int64_t p = p_before; p < p_after; ++p) {
      const int32_t page = kv->fifo.front();
      kv->fifo.pop_front();
      const int32_t idx = static_cast<int32_t>(s * maxp + p);
      kv->table[idx] = page;
      upd.emplace_back(idx, page);
    }
    kv->n_int2[s] += n_evict;
  }
  if (kv->plan_only) return OSCAR_OK;
  hipStream_t st = as_stream(stream);
  rc = push_table(kv, upd, st);
  if (rc) return rc;
  for (int c0 = 0; c0 < n_seqs; c0 += CHUNK) {
    EvictArgs a{};
    a.pool = static_cast<uint8_t*>(kv->desc.pool);
    a.ring = static_cast<uint16_t*>(kv->desc.ring);
    a.page_table = kv->desc.page_table;
    a.hkv = kv->desc.num_kv_heads;
    a.max_pages = kv->desc.max_pages_per_seq;
    a.n_evict = n_evict;
    a.n_seqs = std::min(CHUNK, n_seqs - c0);
    for (int i = 0; i < a.n_seqs; ++i) a.seqs[i] = plan[c0 + i];
    hipError_t e = launch_evict(a, st);
    if (e != hipSuccess) return hip_fail_committed(kv, e, "oscar_kv_evict_window: launch");
  }
  return OSCAR_OK;
}

int oscar_kv_decode_write(oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const void* k, const void* v,
                          void* stream) {
  int rc = check_step_write(kv, seq_ids, n_seqs, k, v, "oscar_kv_decode_write");
  if (rc) return rc;
  std::vector<std::pair<int32_t, int32_t>> upd;
  std::vector<StepSeq> plan = commit_step_write(kv, seq_ids, n_seqs, upd);
  if (kv->plan_only) return OSCAR_OK;
  hipStream_t st = as_stream(stream);
  rc = push_table(kv, upd, st);
  if (rc) return rc;
  for (int c0 = 0; c0 < n_seqs; c0 += CHUNK) {
    const StepArgs a = step_args(kv, k, v, plan, c0, std::min(CHUNK, n_seqs - c0));
    hipError_t e = launch_step_write(a, st);
    if (e != hipSuccess) return hip_fail_committed(kv, e, "oscar_kv_decode_write: launch");
  }
  return OSCAR_OK;
}

int oscar_decode_workspace_bytes(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, size_t* bytes) {
  if (!kv || !bytes) { set_error("oscar_decode_workspace_bytes: null argument"); return OSCAR_E_ARG; }
  int rc = check_seqs(kv, seq_ids, n_seqs);
  if (rc) return rc;
  *bytes = workspace_bytes_for(kv, n_seqs, current_state(kv, seq_ids, n_seqs));
  return OSCAR_OK;
}

int oscar_decode_attn(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const void* q, float sm_scale,
                      float* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(kv, seq_ids, n_seqs, q, sm_scale, out, ws, "oscar_decode_attn");
  if (rc) return rc;
  size_t need = 0;
  rc = oscar_decode_workspace_bytes(kv, seq_ids, n_seqs, &need);
  if (rc) return rc;
  if (ws_bytes < need) {
    set_error("oscar_decode_attn: workspace %zu < %zu bytes", ws_bytes, need);
    return OSCAR_E_WORKSPACE;
  }
  if (kv->plan_only) return OSCAR_OK;
  return launch_decode(kv, seq_ids, n_seqs, nullptr, q, sm_scale, out, ws, as_stream(stream), "oscar_decode_attn");
}

int oscar_decode_step_workspace_bytes(const oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, size_t* bytes) {
  if (!kv || !bytes) { set_error("oscar_decode_step_workspace_bytes: null argument"); return OSCAR_E_ARG; }
  int rc = check_seqs(kv, seq_ids, n_seqs);
  if (rc) return rc;
  // the attention runs on the state after the step's write
  *bytes = workspace_bytes_for(kv, n_seqs, state_after_step(kv, seq_ids, n_seqs));
  return OSCAR_OK;
}

int oscar_decode_step(oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const void* k, const void* v,
                      const void* q, float sm_scale, float* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_step_write(kv, seq_ids, n_seqs, k, v, "oscar_decode_step");
  if (rc) return rc;
  rc = check_decode(kv, seq_ids, n_seqs, q, sm_scale, out, ws, "oscar_decode_step");
  if (rc) return rc;
  size_t need = 0;
  rc = oscar_decode_step_workspace_bytes(kv, seq_ids, n_seqs, &need);
  if (rc) return rc;
  if (ws_bytes < need) {
    set_error("oscar_decode_step: workspace %zu < %zu bytes", ws_bytes, need);
    return OSCAR_E_WORKSPACE;
  }
  // ---- commit
  std::vector<std::pair<int32_t, int32_t>> upd;
  std::vector<StepSeq> plan = commit_step_write(kv, seq_ids, n_seqs, upd);
  if (kv->plan_only) return OSCAR_OK;
  hipStream_t st = as_stream(stream);
  rc = push_table(kv, upd, st);
  if (rc) return rc;
  if (kv->decode_kernel == 1) {
    // the reference kernel has no query preparation to share a launch with
    for (int c0 = 0; c0 < n_seqs; c0 += CHUNK) {
      const StepArgs a = step_args(kv, k, v, plan, c0, std::min(CHUNK, n_seqs - c0));
      hipError_t e = launch_step_write(a, st);
      if (e != hipSuccess) return hip_fail_committed(kv, e, "oscar_decode_step: launch");
    }
    rc = launch_decode(kv, seq_ids, n_seqs, nullptr, q, sm_scale, out, ws, st, "oscar_decode_step");
    if (rc == OSCAR_E_HIP) kv->broken = true;
    return rc;
  }
  rc = launch_decode(kv, seq_ids, n_seqs, &plan, q, sm_scale, out, ws, st, "oscar_decode_step", k, v);
  if (rc == OSCAR_E_HIP) kv->broken = true;
  return rc;
}

int oscar_decode_step_noalloc(oscar_kv* kv, const int32_t* seq_ids, int32_t n_seqs, const void* k, const void* v,
                              const void* q, float sm_scale, float* out, void* stream) {
  int rc = check_step_write(kv, seq_ids, n_seqs, k, v, "oscar_decode_step_noalloc");
  if (rc) return rc;
  size_t need = 0;
  rc = oscar_decode_step_workspace_bytes(kv, seq_ids, n_seqs, &need);
  if (rc) return rc;
  if (need > OSCAR_NOALLOC_SCRATCH_BYTES) {
    set_error("oscar_decode_step_noalloc: the step needs %zu bytes of scratch > %u (use oscar_decode_step with a "
              "workspace)", need, OSCAR_NOALLOC_SCRATCH_BYTES);
    return OSCAR_E_WORKSPACE;
  }
  void* ws = nullptr;  // plan-only stores enqueue nothing and take no workspace
  if (!kv->plan_only) {
    const hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess) return hip_fail(e, "oscar_decode_step_noalloc: scratch address");
  }
  return oscar_decode_step(kv, seq_ids, n_seqs, k, v, q, sm_scale, out, ws, OSCAR_NOALLOC_SCRATCH_BYTES, stream);
}

int oscar_kv_seq_info(const oscar_kv* kv, int32_t seq, int64_t* len, int64_t* n_int2) {
  if (!kv || seq < 0 || seq >= kv->desc.max_seqs) { set_error("oscar_kv_seq_info: bad handle or seq"); return OSCAR_E_ARG; }
  if (len) *len = kv->len[seq];
  if (n_int2) *n_int2 = kv->n_int2[seq];
  return OSCAR_OK;
}

int oscar_kv_get_page_table(const oscar_kv* kv, int32_t* host_out) {
  if (!kv || !host_out) { set_error("oscar_kv_get_page_table: null argument"); return OSCAR_E_ARG; }
  std::memcpy(host_out, kv->table.data(), kv->table.size() * sizeof(int32_t));
  return OSCAR_OK;
}

int oscar_kv_free_pages(const oscar_kv* kv, int32_t* count, int32_t* host_out) {
  if (!kv) { set_error("oscar_kv_free_pages: null handle"); return OSCAR_E_ARG; }
  if (count) *count = static_cast<int32_t>(kv->fifo.size());
  if (host_out) std::copy(kv->fifo.begin(), kv->fifo.end(), host_out);
  return OSCAR_OK;
}

int oscar_kv_reset_seq(oscar_kv* kv, int32_t seq, void* stream) {
  if (!kv || seq < 0 || seq >= kv->desc.max_seqs) { set_error("oscar_kv_reset_seq: bad handle or seq"); return OSCAR_E_ARG; }
  if (int rc = check_usable(kv, "oscar_kv_reset_seq")) return rc;
  const int64_t maxp = kv->desc.max_pages_per_seq;
  const int64_t pages = ceil_div(kv->n_int2[seq], kPage);
  std::vector<std::pair<int32_t, int32_t>> upd;
  for (int64_t p = 0; p < pages; ++p) {
    const int32_t idx = static_cast<int32_t>(seq * maxp + p);
    kv->fifo.push_back(kv->table[idx]);
    kv->table[idx] = -1;
    upd.emplace_back(idx, -1);
  }
  kv->len[seq] = 0;
  kv->n_int2[seq] = 0;
  return push_table(kv, upd, as_stream(stream));
}

int oscar_kv_set_decode_deterministic(oscar_kv* kv, int32_t on) {
  if (!kv || (on != 0 && on != 1)) { set_error("oscar_kv_set_decode_deterministic: on must be 0 or 1"); return OSCAR_E_ARG; }
  kv->deterministic = on;
  return OSCAR_OK;
}

int oscar_kv_set_decode_kernel(oscar_kv* kv, int32_t kernel) {
  if (!kv || kernel < 0 || kernel > 1) { set_error("oscar_kv_set_decode_kernel: kernel must be 0 or 1"); return OSCAR_E_ARG; }
  kv->decode_kernel = kernel;
  return OSCAR_OK;
}

int oscar_kv_set_timing(oscar_kv* kv, int32_t enable) {
  if (!kv) { set_error("oscar_kv_set_timing: null handle"); return OSCAR_E_ARG; }
  if (kv->plan_only) { set_error("oscar_kv_set_timing: plan-only store"); return OSCAR_E_STATE; }
  for (int k = 0; k < 2; ++k) {
    for (hipEvent_t ev : kv->timing_ev[k]) (void)hipEventDestroy(ev);
    kv->timing_ev[k].clear();
    kv->timing_used[k] = 0;
  }
  if (!enable) return OSCAR_OK;
  for (int k = 0; k < 2; ++k) {
    std::vector<hipEvent_t> evs(2 * OSCAR_TIMING_PAIRS, nullptr);
    for (size_t i = 0; i < evs.size(); ++i) {
      // timing-only events: no system-scope fence (no cache writeback/invalidate around the kernel)
      const hipError_t e = hipEventCreateWithFlags(&evs[i], hipEventDisableSystemFence);
      if (e != hipSuccess) {
        for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(evs[j]);
        if (k == 1) {
          for (hipEvent_t ev : kv->timing_ev[0]) (void)hipEventDestroy(ev);
          kv->timing_ev[0].clear();
        }
        return hip_fail(e, "oscar_kv_set_timing: hipEventCreate");
      }
    }
    kv->timing_ev[k] = std::move(evs);
  }
  return OSCAR_OK;
}

int oscar_kv_read_timing(oscar_kv* kv, int32_t kernel, int32_t* launches, double* total_ms, float* each_ms) {
  if (!kv || !launches || !total_ms || kernel < 0 || kernel > 1) {
    set_error("oscar_kv_read_timing: null argument or unknown kernel");
    return OSCAR_E_ARG;
  }
  if (kv->timing_ev[kernel].empty()) { set_error("oscar_kv_read_timing: timing is off"); return OSCAR_E_STATE; }
  double sum = 0.0;
  for (int32_t i = 0; i < kv->timing_used[kernel]; ++i) {
    hipError_t e = hipEventSynchronize(kv->timing_ev[kernel][2 * i + 1]);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, kv->timing_ev[kernel][2 * i], kv->timing_ev[kernel][2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "oscar_kv_read_timing");
    sum += ms;
    if (each_ms) each_ms[i] = ms;
  }
  *launches = kv->timing_used[kernel];
  *total_ms = sum;
  kv->timing_used[kernel] = 0;
  return OSCAR_OK;
}

int oscar_kv_set_decode_split(oscar_kv* kv, int32_t pages_per_split) {
  if (!kv || pages_per_split < 0) { set_error("oscar_kv_set_decode_split: bad argument"); return OSCAR_E_ARG; }
  kv->pages_per_split = pages_per_split;
  return OSCAR_OK;
}

}  // extern "C"
