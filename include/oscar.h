/*
 * oscar.h - C ABI of liboscar: an INT2 paged KV cache with a BF16 attention-sink
 * region and a BF16 recent window, its write path, its window-eviction
 * requantizer and a fused split-K GQA decode-attention read path, for AMD
 * Instinct MI355X (gfx950).
 *
 * Sources (public pages describing OSCAR, "Offline Spectral Covariance-Aware
 * Rotation"):
 *   [A] axbrief, "Together AI's OSCAR breaks the 2-bit KV cache accuracy
 *       barrier" - sections "Together AI, INT2 KV 캐시 시스템 'OSCAR' 공개"
 *       (mixed-precision paged INT2 cache, BF16 sink + recent window, 0.24 %
 *       BF16 at 128K) and "어텐션 통계 기반 회전과 Triton 커널의 결합"
 *       (R_K = U_Q H P_br from the query covariance, clipping c_K = 0.96 /
 *       c_V = 0.92, per-token asymmetric INT2 with 64-channel groups, one
 *       fused read pass: unpack, dequantize, undo rotation, attend; R_V folded
 *       into the projection weights offline).
 *   [B] techllm, "KV cache compression: TurboQuant, OSCAR, EpiCache" - section
 *       "OSCAR — INT2를 실전으로 끌어내린 캘리브레이션 회전" (Hadamard +
 *       bit-reversal spread, recent tokens BF16 / old history INT2).
 *
 * Conventions shared by every call
 *   - Row vectors: a key k is stored rotated as k' = k . R_K; the decode query
 *     is rotated the same way (q' = q . R_K), which gives the same scores as
 *     undoing the rotation on every key ([A], rotation section) because R_K is
 *     orthogonal.
 *   - Values arrive already rotated by R_V ([A]: R_V is absorbed into the value
 *     and output projections offline) and are stored as given; outputs are in
 *     that same basis.
 *   - Query head h reads KV head h / (Hq / Hkv).
 *   - Device pointers are plain HIP device addresses; streams are hipStream_t
 *     passed as void* (NULL = the default stream).  Every device action is
 *     enqueued on that stream in call order; no call synchronizes the device.
 *   - The caller owns every device buffer (pool, ring, page table, rotation,
 *     workspace, inputs, outputs) and keeps it alive until the stream has
 *     passed the call.  The library allocates host memory only (the handle
 *     and its mirror of the page table), never device memory.
 *   - Errors: every call returns OSCAR_OK (0) or a negative status.  A call
 *     that fails validation changes nothing; oscar_last_error() returns a
 *     message for the calling thread.  OSCAR_E_HIP (a HIP runtime call or launch
 *     failed) from a call that changes the store (write, evict, decode-step
 *     write, decode step, reset) comes after the call has moved its host
 *     bookkeeping, so the device state may lag it: the handle is then marked
 *     unusable and every later call on it returns OSCAR_E_STATE; destroy it and
 *     create a new store.  OSCAR_E_HIP from oscar_decode_attn leaves the store
 *     as it was.  Faults inside kernels surface at the caller's next
 *     synchronization.
 *   - One handle must not be used from two host threads at once.
 *
 * Fixed shape (the workloads' and the pages' parameters):
 *   head_dim 128, channel group 64, 64 tokens per page, 64 sink tokens,
 *   256-token recent window, c_K = 0.96, c_V = 0.92.
 */
#ifndef OSCAR_H
#define OSCAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSCAR_HEAD_DIM        128
#define OSCAR_GROUP           64
#define OSCAR_PAGE_TOKENS     64
#define OSCAR_SINK_TOKENS     64
#define OSCAR_WINDOW_TOKENS   256
#define OSCAR_RING_SLOTS      (OSCAR_SINK_TOKENS + OSCAR_WINDOW_TOKENS)
#define OSCAR_HEAD_BLOCK      5120   /* bytes of one KV head in one page */
#define OSCAR_ROT_HEAD_BYTES  164352 /* bytes of one KV head's rotation block */
#define OSCAR_MAX_GQA         8      /* Hq / Hkv must be 1, 2, 4 or 8 */

enum {
    OSCAR_OK = 0,
    OSCAR_E_ARG = -1,           /* bad argument: null pointer, shape, range, duplicate seq id */
    OSCAR_E_NOPAGE = -2,        /* the free-page FIFO cannot supply every page the call needs */
    OSCAR_E_WINDOW_FULL = -3,   /* an append would hold more than 256 window tokens */
    OSCAR_E_WINDOW_SHORT = -4,  /* eviction asks for more tokens than the window holds */
    OSCAR_E_NUMERIC = -5,       /* non-finite calibration input or eigensolver failure */
    OSCAR_E_HIP = -6,           /* a HIP runtime call or kernel launch failed */
    OSCAR_E_WORKSPACE = -7,     /* decode workspace smaller than oscar_decode_workspace_bytes */
    OSCAR_E_STATE = -8          /* the call does not fit the sequence's state (e.g. empty sequence), or
                                   the handle is unusable after an OSCAR_E_HIP */
};

/* Set in oscar_kv_desc.flags: keep every piece of host bookkeeping (page table
 * mirror, FIFO, lengths) but enqueue no device work and accept NULL device
 * pointers.  For capacity planning and for testing the allocator on a host
 * without a GPU. */
#define OSCAR_FLAG_PLAN_ONLY 1

typedef struct oscar_kv oscar_kv;

/*
 * One attention layer's mixed-precision paged store ([A] Release section: the
 * INT2 cache stays a paged-attention cache, BF16 sink + recent window, INT2
 * history).
 *
 * pool        device, num_pages * num_kv_heads * OSCAR_HEAD_BLOCK bytes.  Page p,
 *             KV head h is the 5120-byte block at (p * num_kv_heads + h) * 5120:
 *               [   0, 2048) key codes, [2048, 4096) value codes: 2 bits per code,
 *                            512 little-endian 32-bit words each;
 *               [4096, 5120) metadata, 16 bytes per token j at 4096 + 16 j:
 *                            fp16 {sK0, loK0, sK1, loK1, sV0, loV0, sV1, loV1}
 *                            (scale and minimum of channel groups 0-63, 64-127).
 *             Key code of token j, channel c:
 *               t = j/16, n = j%16, g = c/64, kq = (c%64)/16, u = c%16,
 *               word = 256*(t/2) + 4*(16*kq + n) + 2*(t%2) + g,
 *               bit  = 8*(u%4) + 2*(u/4).
 *             Value code of token j, channel c:
 *               ct = c/16, n = c%16, s = j/32, kq = (j%32)/8, kk = j%8,
 *               word = 256*(ct/4) + 4*(16*kq + n) + ct%4,
 *               bit  = 2*(4*s + kk/2) + 16*(kk%2).
 *             Slots of tokens not yet written in a page are zero.
 * ring        device bf16, [max_seqs][num_kv_heads][2 (K,V)][320][128].  Slot p < 64
 *             holds sink position p; window position p >= 64 sits in slot
 *             64 + (p - 64) % 256.  Keys are stored rotated (bf16 of k . R_K).
 * page_table  device int32 [max_seqs][max_pages_per_seq]: physical page of each
 *             64-token INT2 page, -1 where none.  INT2 index i (position 64 + i)
 *             lives in page page_table[seq][i / 64], slot i % 64.
 * rot         device, num_kv_heads * OSCAR_ROT_HEAD_BYTES bytes, written by
 *             oscar_kv_set_rotation: per KV head R_K fp32 [128][128] followed by
 *             three bf16 [128][128] terms of R_K^T (term t, output channel c,
 *             input channel i; r0 = bf16(R^T), r1 = bf16(R^T - r0),
 *             r2 = bf16(R^T - r0 - r1), whose sum is R^T within 2^-24 of it),
 *             then fp32 [128] -(mu . R_K) for the key mean mu set by
 *             oscar_kv_set_key_mean (+0 where that is zero; all +0 without a
 *             mean).
 */
typedef struct {
    int32_t num_q_heads;        /* Hq, a multiple of num_kv_heads with Hq/Hkv <= 8 */
    int32_t num_kv_heads;       /* Hkv >= 1 */
    int32_t max_seqs;           /* sequence slots; seq ids are 0 .. max_seqs-1 */
    int32_t max_pages_per_seq;  /* page-table row length */
    int32_t num_pages;          /* pages in the pool */
    int32_t flags;              /* 0 or OSCAR_FLAG_PLAN_ONLY */
    void *pool;
    void *ring;
    int32_t *page_table;
    void *rot;
} oscar_kv_desc;

/*
 * Key rotation from calibration queries, on the host, in fp64 ([A] rotation
 * section: R_K = U_Q . H_Had . P_br, U_Q the eigenvectors of the query
 * covariance C_Q = (1/N) sum_n q_n^T q_n; [B]: Hadamard + bit reversal).
 *
 * q        host fp32 [n][d], row n is one query (pool every query head that
 *          reads the KV head).  No mean is subtracted.
 * d        must be 128.
 * rot_out  host fp32 [d][d], row-major, R_K = U . H . P with U's columns in
 *          descending eigenvalue order, each column's largest-magnitude entry
 *          positive, H the Sylvester Hadamard matrix / sqrt(d), and
 *          (x . P)_j = x_{bitreverse(j)}.
 * eig_out  host fp64 [d], descending eigenvalues of C_Q, or NULL.
 * Errors: OSCAR_E_ARG (null pointer, n < 1, d != 128), OSCAR_E_NUMERIC
 * (non-finite input, eigensolver did not converge).  Writes nothing on error.
 */
int oscar_calibrate_host(const float *q, int64_t n, int32_t d, float *rot_out, double *eig_out);

/*
 * Offline value-rotation calibration ([A] rotation section: R_V = U_S . H_Had .
 * P_br with U_S the eigenvectors of C_S = (1/N) V^T S^T S V), on the host in fp64.
 *
 * s        host fp32 [n_q][n_tok]: attention probabilities of n_q calibration
 *          queries over n_tok calibration tokens (rows normally sum to 1; pool
 *          the queries of every q head that reads this KV head).
 * v        host fp32 [n_tok][d]: the (unrotated) values of those tokens.
 * d        must be 128.
 * rot_out  host fp32 [d][d], row-major R_V (values are stored as v . R_V).
 * eig_out  host fp64 [d] eigenvalues of C_S, descending; may be NULL.
 * C_S is accumulated as the second moment of the attention outputs o_n = s_n V.
 * Eigenvector order and signs, H and P_br as for oscar_calibrate_host.
 * Errors: OSCAR_E_ARG (null, sizes), OSCAR_E_NUMERIC (non-finite input,
 * eigensolver failure).
 */
int oscar_calibrate_value_host(const float *s, const float *v, int64_t n_q, int64_t n_tok, int32_t d,
                               float *rot_out, double *eig_out);

/*
 * Absorb R_V into a layer's projections, in place, on the host ([A] rotation
 * section: R_V is folded offline into the value/output projections, so the cache
 * stores rotated values at no runtime cost and oscar_decode_attn's output, which
 * is in the R_V basis, is un-rotated by the output projection).
 *
 * w_v  host fp32 [d_model][num_kv_heads * 128] row-major (x . w_v = values);
 *      columns of KV head h become w_v[:, h block] . R_V[h].
 * w_o  host fp32 [num_q_heads * 128][d_model] row-major (o . w_o = output);
 *      rows of q head j become R_V[h]^T . w_o[j block], h = j / (Hq / Hkv).
 * r_v  host fp32 [num_kv_heads][128][128].
 * Products are accumulated in fp64 and rounded to fp32.
 * Errors: OSCAR_E_ARG (null, head counts), OSCAR_E_NUMERIC (non-finite r_v).
 */
int oscar_fold_value_rotation(int32_t d_model, int32_t num_q_heads, int32_t num_kv_heads, const float *r_v,
                              float *w_v, float *w_o);

/* Bytes the caller must allocate for each device buffer of a store with this
 * descriptor (device pointers in desc are ignored).  Any output may be NULL. */
int oscar_kv_buffer_bytes(const oscar_kv_desc *desc, size_t *pool, size_t *ring,
                          size_t *page_table, size_t *rot);

/*
 * Create a store.  free_pages (host, n_free entries, distinct, each in
 * [0, num_pages)) is the initial FIFO of free physical pages.  Unless
 * OSCAR_FLAG_PLAN_ONLY is set, fills the device page table with -1 on stream.
 * Every sequence starts empty.  *out is set only on success.
 */
int oscar_kv_create(const oscar_kv_desc *desc, const int32_t *free_pages, int32_t n_free,
                    void *stream, oscar_kv **out);

/*
 * Upload R_K for every KV head (host fp32 [num_kv_heads][128][128], row-major,
 * as produced by oscar_calibrate_host) into desc.rot on stream, with its bf16
 * three-term split.  Must be called before the first write or decode.
 * Errors: OSCAR_E_ARG (null), OSCAR_E_NUMERIC (non-finite entry).
 */
int oscar_kv_set_rotation(oscar_kv *kv, const float *rot_host, void *stream);

/*
 * Append n_new tokens to each listed sequence ([A] rotation section: each new
 * key is rotated by R_K, clipped with c_K, quantized per token to asymmetric
 * INT2 in 64-channel groups; values likewise with c_V, unrotated).
 *
 * seq_ids  host int32 [n_seqs], distinct.
 * k, v     device bf16 [n_seqs][n_new][num_kv_heads][128], token order = position
 *          order.
 * Routing: into an empty sequence of final length L, positions < 64 go to the
 * BF16 sink, positions 64 .. L-257 are quantized straight to INT2 (from the
 * fp32 rotated key) and the last min(L-64, 256) positions go to the BF16
 * window.  Into a non-empty sequence, positions < 64 go to the sink and the
 * rest to the window; when they do not fit (the sink and window hold 320
 * tokens) and oscar_kv_set_write_evicts is on, each token that does not fit
 * first moves the oldest window token into INT2, as oscar_kv_evict_window
 * would (from its stored bf16 copy): the stored state equals that of writing
 * the tokens one at a time with an eviction whenever the window is full
 * (techllm "KV cache compression", OSCAR section: recent tokens BF16, older
 * history INT2).  Pages are taken from the FIFO in seq_ids order, ascending
 * within a sequence.
 * Errors: OSCAR_E_ARG, OSCAR_E_WINDOW_FULL (a non-empty sequence's window
 * would exceed 256 tokens and evicting writes are off: evict first),
 * OSCAR_E_NOPAGE (FIFO too short or a sequence would exceed
 * max_pages_per_seq); nothing is changed on error.
 */
int oscar_kv_write(oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs, int32_t n_new,
                   const void *k, const void *v, void *stream);

/* Output precision of oscar_decode_attn and oscar_decode_step: on = 1 writes
 * `out` as bf16 (round to nearest even of the fp32 result; the pointer then
 * addresses 2-byte elements, same [n_seqs][num_q_heads][128] order), on = 0
 * (default) as fp32.  For engines whose output projection reads bf16.
 * Errors: OSCAR_E_ARG. */
int oscar_kv_set_output_bf16(oscar_kv *kv, int32_t on);

/* Evicting writes (chunked prefill): on = 1 lets oscar_kv_write overflow a
 * non-empty sequence's window, evicting as it goes (see above); on = 0
 * (default) returns OSCAR_E_WINDOW_FULL instead.  Errors: OSCAR_E_ARG. */
int oscar_kv_set_write_evicts(oscar_kv *kv, int32_t on);

/*
 * Move the n_evict oldest window tokens of each listed sequence into INT2
 * ([A]/[B]: old history is INT2, recent tokens BF16): each is quantized from
 * its stored bf16 key (already rotated) and value, into INT2 index n_int2,
 * n_int2 + 1, ...; a page is taken from the FIFO whenever the index is a
 * multiple of 64 (sequences in seq_ids order).
 * Errors: OSCAR_E_ARG, OSCAR_E_WINDOW_SHORT, OSCAR_E_NOPAGE.
 */
int oscar_kv_evict_window(oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs, int32_t n_evict,
                          void *stream);

/*
 * The decode step's write in one launch: for each listed (non-empty) sequence,
 * when its window holds 256 tokens, move the oldest one into INT2 (as
 * oscar_kv_evict_window with n_evict = 1, taking a page from the FIFO when the
 * INT2 index is a multiple of 64), then append one token (as oscar_kv_write with
 * n_new = 1).  The stored state equals that of the two calls.  k, v: bf16 device
 * arrays [n_seqs][num_kv_heads][128], row i for seq_ids[i].
 * Errors: OSCAR_E_ARG, OSCAR_E_STATE (an empty sequence, or no rotation),
 * OSCAR_E_NOPAGE; nothing is changed on error.
 */
int oscar_kv_decode_write(oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs, const void *k,
                          const void *v, void *stream);

/* Device workspace bytes oscar_decode_attn needs for these sequences in their
 * current state (split-K partials, prepared queries, per-split page counters). */
int oscar_decode_workspace_bytes(const oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs,
                                 size_t *bytes);

/*
 * One decode step of GQA attention for each listed sequence over everything
 * it stores ([A] rotation section: one fused pass unpacks, dequantizes,
 * handles the rotation and attends, with no extra memory traffic).
 *
 * q         device bf16 [n_seqs][num_q_heads][128] (unrotated queries).
 * sm_scale  softmax scale (1/sqrt(128) for standard attention).
 * out       device fp32 [n_seqs][num_q_heads][128], softmax(sm_scale q k^T) v in
 *           the R_V basis (bf16 [n_seqs][num_q_heads][128] when
 *           oscar_kv_set_output_bf16 is on).
 * ws        device workspace of at least oscar_decode_workspace_bytes bytes.
 * Errors: OSCAR_E_ARG, OSCAR_E_STATE (an empty sequence), OSCAR_E_WORKSPACE.
 */
int oscar_decode_attn(const oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs, const void *q,
                      float sm_scale, float *out, void *ws, size_t ws_bytes, void *stream);

/* Device workspace bytes oscar_decode_step needs for these sequences: the
 * attention's workspace on the state after the step's write. */
int oscar_decode_step_workspace_bytes(const oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs,
                                      size_t *bytes);

/*
 * One whole decode step per listed (non-empty) sequence in one call: the
 * decode-step write (as oscar_kv_decode_write: evict the oldest window token
 * when the window holds 256, then append k, v) followed by decode attention
 * over everything stored, the new token included (as oscar_decode_attn).  The
 * stored state and the output equal those of the two calls ([A] rotation
 * section: new tokens are rotated and quantized on write, and the read path is
 * one fused pass; the write shares the launch of the query preparation).
 * k, v      device bf16 [n_seqs][num_kv_heads][128], row i for seq_ids[i].
 * q         device bf16 [n_seqs][num_q_heads][128] (unrotated queries).
 * sm_scale  softmax scale (1/sqrt(128) for standard attention).
 * out       device fp32 [n_seqs][num_q_heads][128], in the R_V basis (bf16 when
 *           oscar_kv_set_output_bf16 is on).
 * ws        device workspace of at least oscar_decode_step_workspace_bytes bytes.
 * The caller owns every buffer; calls are enqueued on stream in order.
 * Errors: OSCAR_E_ARG, OSCAR_E_STATE (an empty sequence, or no rotation),
 * OSCAR_E_NOPAGE, OSCAR_E_WORKSPACE; nothing is changed on error.
 */
int oscar_decode_step(oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs, const void *k, const void *v,
                      const void *q, float sm_scale, float *out, void *ws, size_t ws_bytes, void *stream);

/*
 * oscar_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the step's split partials, prepared queries
 * and page-group counters live in a device array inside the library,
 * OSCAR_NOALLOC_SCRATCH_BYTES bytes per GPU, held from the library's load until
 * the process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); its first call on a device looks the array's address up.
 * Arguments, results and errors as oscar_decode_step; OSCAR_E_WORKSPACE when
 * the step needs more than OSCAR_NOALLOC_SCRATCH_BYTES (what
 * oscar_decode_step_workspace_bytes reports), OSCAR_E_HIP when the array's
 * address cannot be looked up (nothing is changed then).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (two streams, two
 * threads, two handles) race and must be ordered by the caller.
 */
#define OSCAR_NOALLOC_SCRATCH_BYTES (32u << 20)
int oscar_decode_step_noalloc(oscar_kv *kv, const int32_t *seq_ids, int32_t n_seqs, const void *k,
                              const void *v, const void *q, float sm_scale, float *out, void *stream);

/* Length and INT2 token count of one sequence. */
int oscar_kv_seq_info(const oscar_kv *kv, int32_t seq, int64_t *len, int64_t *n_int2);

/* Copy of the host mirror of the page table, int32 [max_seqs][max_pages_per_seq]. */
int oscar_kv_get_page_table(const oscar_kv *kv, int32_t *host_out);

/* Number of free pages and the FIFO contents (host int32, may be NULL). */
int oscar_kv_free_pages(const oscar_kv *kv, int32_t *count, int32_t *host_out);

/* Empty one sequence: its pages go to the FIFO tail in ascending logical order;
 * its device page-table row is reset to -1 on stream. */
int oscar_kv_reset_seq(oscar_kv *kv, int32_t seq, void *stream);

/* Key-mean subtraction on write (gist.science summary of OptR, section
 * "해결책: OptR (출력 인지 회전)", step 1: keys are centred by a per-head mean
 * before the rotation; a query's scores all move by the same q . mu, which the
 * softmax cancels, so attention is unchanged while the INT2 groups see
 * centred keys).  mean: host fp32 [num_kv_heads][128], finite, or NULL to
 * remove the mean.  Every key written after the call (multi-token writes,
 * appends, decode-step writes) is stored as (k - mu) . R_K; keys already in
 * the cache keep the mean they were written with, so set it before the first
 * write of a sequence.  The mean is kept on the host and, once a rotation is
 * set, uploaded on stream (the call waits for the upload); setting a new
 * rotation re-applies it.  OSCAR_E_ARG for a non-finite entry. */
int oscar_kv_set_key_mean(oscar_kv *kv, const float *mean, void *stream);

/* Decode tuning: pages_per_split = 0 picks a split size from the batch. */
int oscar_kv_set_decode_split(oscar_kv *kv, int32_t pages_per_split);

/* Decode reproducibility.  on = 0 (default): the INT2 splits of one (sequence,
 * KV head) share their pages at run time (a split that finishes early takes page
 * groups of the others), which evens out the finishing times of the work-groups;
 * which pages land in which partial record then varies between calls, and so do
 * the outputs, by the rounding of p * s to the fp16 pair relative to each record's
 * running maximum (about 1e-5 relative, bounded by the same 1e-3 parity bound).
 * on = 1: every split covers a fixed page range, and repeated calls on the same
 * state give bitwise identical outputs for a given split size.  The reference
 * kernel (1) is always deterministic.  OSCAR_E_ARG unless on is 0 or 1. */
int oscar_kv_set_decode_deterministic(oscar_kv *kv, int32_t on);

/* Decode kernel: 0 (default) = the matrix-core kernel (i8 MFMA for q.k on the raw
 * codes, f16 MFMA for p.v); 1 = the reference-grade kernel that dequantizes every
 * element in fp32 (slow; kept as an independent cross-check). */
int oscar_kv_set_decode_kernel(oscar_kv *kv, int32_t kernel);

/* Kernel timing (measurement aid).  enable = 1 creates OSCAR_TIMING_PAIRS HIP event
 * pairs per timed kernel (timing-only: no system-scope fence on record); from then
 * on every call records one pair around each launch of its main kernel, on the
 * call's stream, until that kernel's pairs are used up (further launches go
 * untimed):
 *   OSCAR_TIMED_DECODE  the split kernel of oscar_decode_attn (not the query
 *                       preparation or the combine);
 *   OSCAR_TIMED_WRITE   the write kernel of oscar_kv_write (not the page-table
 *                       upload).
 * The recorded events sit between that kernel and its neighbours on the stream:
 * each adds a few microseconds of gap on the GPU (kernels otherwise start back to
 * back) and the measured interval includes the kernel's dispatch latency, so time
 * whole calls with timing off.  enable = 0 destroys the events.  Returns OSCAR_E_ARG on a null handle,
 * OSCAR_E_STATE for a plan-only store, OSCAR_E_HIP if event creation fails (then
 * timing stays off). */
#define OSCAR_TIMING_PAIRS 4096
#define OSCAR_TIMED_DECODE 0
#define OSCAR_TIMED_WRITE  1
int oscar_kv_set_timing(oscar_kv *kv, int32_t enable);

/* Waits for the pairs recorded for `kernel` (OSCAR_TIMED_*), writes the number of
 * timed launches to *launches, their summed duration in milliseconds to
 * *total_ms and, when each_ms is not NULL, each launch's duration in launch order
 * to each_ms[0 .. *launches - 1] (room for OSCAR_TIMING_PAIRS entries), and frees
 * those pairs for reuse.  OSCAR_E_ARG for a null argument or an unknown kernel,
 * OSCAR_E_STATE when timing is off. */
int oscar_kv_read_timing(oscar_kv *kv, int32_t kernel, int32_t *launches, double *total_ms, float *each_ms);

const char *oscar_last_error(void);
void oscar_kv_destroy(oscar_kv *kv);

#ifdef __cplusplus
}
#endif
#endif /* OSCAR_H */
