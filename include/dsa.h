/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) prefill hot path for one
 * context-parallel (CP) rank, on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [xLLM-CP]    "feat: DeepSeek-V4 DSA context-parallel on NPU" (xLLM pull request page)
 *   [CP-blog]    "[DeepSeek v3.2] context parallel explained" (blog post on SGLang's NSA prefill CP)
 *   [CP-gathers] "The role of the two all-gathers in NSA prefill CP" (SGLang design note)
 *
 * The rank owns a slice of the flattened query stream -- contiguous ("in-seq") or round-robin
 * (token t on rank t % cp_size) -- and attends over the full KV stream in logical order, which
 * every rank holds ([xLLM-CP] Non-goals and Design key points; [CP-blog] Part 3 step C).
 *
 * Conventions for every entry point:
 *   - Tensor pointers marked "device" are HIP device pointers owned by the caller. The library
 *     allocates nothing, keeps no pointer after return and never synchronises: each call only
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - Tensors are dense, row-major, contiguous; device pointers must be 16-byte aligned.
 *   - Integers are int32 unless stated. Floating point: see dsa_dtype.
 *   - Return value: DSA_OK, or an error code with a message in dsa_last_error() (per thread).
 *     Argument errors are detected on the host before anything is launched. Inconsistencies
 *     only visible on the device (e.g. cu-seqlens that do not match the row count) are reported
 *     by OR-ing DSA_DEVERR_* bits into *err_flag (device int32, optional) and the offending row
 *     is skipped, so nothing is read out of bounds.
 *   - Checked build: libdsa_checked.so (the same sources compiled with DSA_CHECKED) also verifies,
 *     before each use, every gathered KV / key row id and every data-dependent LDS or output index
 *     the kernels compute (list slots, compacted-row slots, histogram bins, bitmap words, output
 *     positions). A failed check ORs DSA_DEVERR_BOUNDS into *err_flag and skips that access; no
 *     check traps. Its results are those of libdsa.so bit for bit; it is for testing, not speed.
 *   - The library is reentrant; its only state is the per-thread error string.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misalignment, rank out of range ... */
  DSA_ERR_UNSUPPORTED = 2,  /* shape / dtype combination not built into this library       */
  DSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the size query returned   */
  DSA_ERR_HIP = 4           /* a HIP launch failed; dsa_last_error() holds HIP's message   */
} dsa_status;

typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2  /* OCP 8-bit float E4M3FN: bias 7, max 448, no infinities */
} dsa_dtype;

typedef enum {
  DSA_SPLIT_IN_SEQ = 0,      /* rank r owns tokens [r*tpr, (r+1)*tpr) of the padded stream */
  DSA_SPLIT_ROUND_ROBIN = 1  /* rank r owns tokens r, r+cp, r+2cp, ...                     */
} dsa_split;

/* Device-side error bits written to *err_flag. */
#define DSA_DEVERR_QSL_START 0x1      /* query_start_loc[0] != 0                                 */
#define DSA_DEVERR_QSL_ORDER 0x2      /* query_start_loc decreasing                              */
#define DSA_DEVERR_SEQ_LENS 0x4       /* seq_lens[b] < query length of request b                 */
#define DSA_DEVERR_QSL_TOTAL 0x8      /* query_start_loc[B] != num_tokens                        */
#define DSA_DEVERR_ROWS 0x10          /* local cu_seqlens_q[B] != nq (global metadata passed?)   */
#define DSA_DEVERR_EXTENT 0x20        /* a query's causal extent is outside the key buffer       */
#define DSA_DEVERR_INDEX 0x40         /* a selected KV row id is outside [-1, n_rows)            */
#define DSA_DEVERR_BOUNDS 0x80        /* checked build only: an internal index failed its check  */

/* Message describing the last error returned on the calling thread ("" if none). */
const char* dsa_last_error(void);

/* Library version string, for logs. */
const char* dsa_version(void);

/* ------------------------------------------------------------------------------------------
 * Host-only sizing of a rank's share ([xLLM-CP] Implementation §2: num_tokens_pad is the token
 * count rounded up to a multiple of cp_size, tokens_per_rank = num_tokens_pad / cp_size;
 * [CP-blog] §2B and Part 3.1 for the round-robin split).
 *   tokens_per_rank : rows of the rank's local buffer (real tokens first, then pad rows).
 *   n_local_real    : real tokens the rank owns.
 *   num_rows_concat : rows of the rank-concatenated buffer that dsa_rerange reads
 *                     (cp_size*tokens_per_rank when padded, else num_tokens).
 * Any output pointer may be NULL. No device work.
 * ------------------------------------------------------------------------------------------ */
dsa_status dsa_cp_sizes(int32_t num_tokens, int32_t cp_size, int32_t cp_rank, int32_t mode,
                        int32_t pad_to_cp, int32_t* tokens_per_rank, int32_t* n_local_real,
                        int32_t* num_rows_concat);

/* ------------------------------------------------------------------------------------------
 * (1) CP-local metadata ([xLLM-CP] Implementation §2, build of the CP-local metadata; Design,
 * key points: local queries see a right-aligned KV extent and the last rank sees the whole
 * stream; [CP-blog] §2B: after the round-robin scatter the per-rank sequence lengths and
 * cu-seqlens are recomputed; [xLLM-CP] Testing: chunked prefill is part of the functional
 * matrix).
 *
 * In (device): query_start_loc [batch+1] (global cu-seqlens of the flattened query stream),
 *              seq_lens [batch] (KV tokens of each request, >= its query length n_b).
 * Chunked prefill: request b carries P_b = seq_lens[b] - n_b cached tokens. Its KV segment is
 * seq_lens[b] rows long, prefix first, and the segments follow one another in request order
 * (segment b starts at row sum_{b'<b} seq_lens[b']). Query g (0-based) of request b sits at
 * KV position P_b + g. Pure prefill is P_b = 0 for every request.
 * Out (device):
 *   local_query_start_loc [batch+1]  cu-seqlens of the rank's real local queries per request
 *   local_seq_lens        [batch]    KV extent seen by the request's last local query
 *                                    (in-seq: P_b + clamp(local_end - qs_b, 0, n_b);
 *                                     round-robin: P_b + last local position + 1, or P_b)
 *   local_kv_start_loc    [batch+1]  KV row where request b starts (in-seq: right-aligned
 *                                    cumsum of local_seq_lens; round-robin: the segment
 *                                    starts, = query_start_loc in pure prefill)
 *   scalars [8]: num_tokens_pad, tokens_per_rank, local_start, local_end, stride (1 or cp),
 *                n_local_real, max_seqlen_q, num_local_reqs
 *   token_map [tokens_per_rank] (optional): global token id of each local row, -1 for pads
 *   err_flag [1] (optional): DSA_DEVERR_QSL_* / DSA_DEVERR_SEQ_LENS bits (a request flagged
 *                            SEQ_LENS is treated as having no prefix)
 * Local query j (0-based) of request b, with n_b = local_query_start_loc[b+1] - [b], sees the
 * keys [local_kv_start_loc[b], local_kv_start_loc[b] + E) with
 *   E = local_seq_lens[b] - (n_b - 1 - j) * stride.
 * `pad_to_cp` only changes how the rank-concatenated buffer is laid out (see dsa_rerange).
 * ------------------------------------------------------------------------------------------ */
dsa_status dsa_build_cp_metadata(const int32_t* query_start_loc, const int32_t* seq_lens,
                                 int32_t batch, int32_t num_tokens, int32_t cp_size,
                                 int32_t cp_rank, int32_t mode, int32_t pad_to_cp,
                                 int32_t* local_query_start_loc, int32_t* local_seq_lens,
                                 int32_t* local_kv_start_loc, int32_t* scalars,
                                 int32_t* token_map, int32_t* err_flag, void* stream);

/* ------------------------------------------------------------------------------------------
 * (2)+(3) Lightning-indexer scores and per-query causal top-k ([xLLM-CP] Design, data-flow
 * step (3) and Implementation §4: the indexer query, weights and top-k use the local rows and
 * local cu-seqlens, the index keys the full stream; Implementation §5: localised indexer
 * metadata, else the top-k collapses to position 0).
 *
 *   score(i, s) = sum_h w[i,h] * max(0, q_hat[i,h,:] . k_hat[kv0(i) + s, :]),  0 <= s < Ev(i)
 *   bf16 / f32: q_hat = q_idx, k_hat = k_idx.
 *   fp8:        q_hat = q_idx * q_scale[i,h], k_hat = k_idx * k_scale[row] (scales > 0).
 *   Ev(i) = E(i) (see dsa_build_cp_metadata), or floor(E(i)/compress_ratio) whole compressed
 *   blocks; -0.0 scores count as +0.0.
 * Top-k of row i: if Ev <= topk every visible key, else the topk best by (score descending,
 * key index ascending). Written to topk_idx[i, 0:topk] as absolute rows
 * kv_row_base + cu_seqlens_kv[b] + s in ascending order, -1 after the last one.
 * With window > 0, topk_idx[i, topk:topk+window] holds the original-token rows
 * window_kv_start[b] + p' for p' in [max(0, p-window+1), p] (p = E(i)-1), -1 padded.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const void* q_idx;            /* device [nq, n_heads, head_dim], dtype `dtype`            */
  const float* q_scale;         /* device [nq, n_heads] (fp8 only, else NULL)               */
  const float* weights;         /* device [nq, n_heads] float32                              */
  const void* k_idx;            /* device [nk, head_dim], dtype `dtype`                      */
  const float* k_scale;         /* device [nk] (fp8 only, else NULL)                         */
  int32_t dtype;                /* dsa_dtype of q_idx and k_idx                              */
  int32_t nq;                   /* local query rows (must equal cu_seqlens_q[batch])         */
  int32_t nk;                   /* key rows in k_idx                                         */
  int32_t n_heads;              /* indexer heads H_i                                         */
  int32_t head_dim;             /* indexer dim D_i                                           */
  int32_t batch;                /* requests B                                                */
  const int32_t* cu_seqlens_q;  /* device [B+1] local_query_start_loc                       */
  const int32_t* seqused_kv;    /* device [B]   local_seq_lens (token units)                 */
  const int32_t* cu_seqlens_kv; /* device [B+1] key-row offset of request b in k_idx          */
  int32_t max_seqlen_kv;        /* host bound on seqused_kv (token units): sizes the score
                                   rows; rows with a larger extent are skipped + flagged     */
  int32_t q_stride;             /* 1 for in-seq, cp_size for round-robin                      */
  int32_t compress_ratio;       /* 1, or the key compression ratio (4)                       */
  int32_t topk;                 /* K >= 1                                                    */
  int32_t kv_row_base;          /* added to emitted top-k rows                               */
  int32_t window;               /* 0, or sliding-window rows appended after the top-k rows   */
  const int32_t* window_kv_start;  /* device [B+1] original-row start of request b (window) */
  int32_t* topk_idx;            /* device out [nq, topk + window] int32                      */
  void* workspace;              /* device scratch of >= dsa_indexer_topk_workspace() bytes   */
  size_t workspace_bytes;
  int32_t* err_flag;            /* device [1] or NULL                                        */
} dsa_indexer_topk_args;

/* Workspace bytes the call needs (0 if the arguments are invalid; see dsa_last_error). */
size_t dsa_indexer_topk_workspace(const dsa_indexer_topk_args* args);

/* Scores then top-k, both on `stream`. Rows with at most `topk` visible keys are taken whole
 * by the top-k, so the indexer computes no scores for them (their workspace row is untouched). */
dsa_status dsa_indexer_topk(const dsa_indexer_topk_args* args, void* stream);

/* The two halves separately, on caller-provided score rows: scores [nq, ld] float32 with
 * ld >= visible(max_seqlen_kv) and ld % 4 == 0; entries past a row's visible count are not
 * written by dsa_indexer_scores and not read by dsa_topk_from_scores. The workspace fields
 * are ignored by these two. */
dsa_status dsa_indexer_scores(const dsa_indexer_topk_args* args, float* scores, int64_t ld,
                              void* stream);
dsa_status dsa_topk_from_scores(const dsa_indexer_topk_args* args, const float* scores,
                                int64_t ld, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): dsa_indexer_topk with the library's own scratch instead
 * of args->workspace (ignored). The scratch is a static 64 MiB device array, one copy per GPU the
 * library runs on, held until the process ends; the call allocates nothing. Every call on a GPU
 * shares that GPU's copy, so calls that overlap on one GPU (other streams, other host threads)
 * race and give wrong results: serialise them. The scratch keeps the previous call's contents;
 * nothing in it needs to start at zero. `stream` must belong to the current device.
 * Errors: those of dsa_indexer_topk; DSA_ERR_WORKSPACE (before any launch) when
 * dsa_indexer_topk_workspace() of the call exceeds 64 MiB (e.g. more than ~16M score entries). */
dsa_status dsa_indexer_topk_noalloc(const dsa_indexer_topk_args* args, void* stream);

/* Measurement hook, for benchmarks and profilers that time the kernels inside one call:
 * dsa_indexer_topk(args, stream), with events[k] recorded on `stream` right before the k-th
 * kernel the call launches and events[n] right after the last one, n = *n_kernels (out), so
 * hipEventElapsedTime(events[k], events[k+1]) is the k-th kernel's time. events are hipEvent_t
 * handles created by the caller (with timing enabled to read durations); kernels past the
 * (n_events - 1)-th run unbracketed. kernel_names (optional, n_events entries) receives static
 * strings naming the kernels. Errors: those of dsa_indexer_topk; DSA_ERR_INVALID_ARG for fewer
 * than 2 events or a NULL event; DSA_ERR_HIP if an event cannot be recorded. */
dsa_status dsa_indexer_topk_timed(const dsa_indexer_topk_args* args, void* stream, void* const* events,
                                  int32_t n_events, int32_t* n_kernels, const char** kernel_names);

/* Measurement hook, for benchmarks that report the graphics clock a run held: enqueues on
 * `stream` one wave that reads the shader-clock counter and the 100 MHz real-time counter, spins
 * for `ticks` real-time ticks (1 .. 1e7, i.e. 10 ns .. 100 ms) and reads both again, writing
 * {clock0, clock1, realtime0, realtime1} to out (device, 4 x uint64). The clock in MHz is
 * 100 * (clock1 - clock0) / (realtime1 - realtime0). DSA_ERR_INVALID_ARG for a NULL out or ticks
 * out of range. */
dsa_status dsa_clock_probe(uint64_t* out, int64_t ticks, void* stream);

/* Measurement hook, for the ceiling of the MLA attention kernel's MFMA rate: enqueues on `stream`
 * 256 workgroups of 64 * 4 * waves_per_simd threads (one or two waves per SIMD); every wave runs
 * iters x 32 dependent 32x32x16 bf16 MFMAs whose A operand comes from LDS in the attention
 * kernel's K form (operand 0: one 16-byte read per lane per MFMA) or V form (operand 1: two 8-byte
 * transposed reads per lane), or from registers (operand 2), reads issued three MFMAs ahead. Wave w
 * of workgroup g writes the shader-clock cycles of its loop to cycles[8 g + w] (device, >= 2048
 * entries; other entries untouched); sink (device, >= 256 x threads floats) receives values that
 * keep the MFMA chain live. The MFMA busy fraction of a SIMD is 32 x iters x 32 x waves_per_simd
 * / cycles (32 cycles per MFMA). DSA_ERR_INVALID_ARG for operand outside 0..2, waves_per_simd
 * outside 1..2, iters outside 1..1e5, or NULL / short buffers. */
dsa_status dsa_lds_mfma_probe(int32_t operand, int32_t waves_per_simd, int32_t iters, uint64_t* cycles,
                              int64_t n_cycles, float* sink, int64_t n_sink, void* stream);

/* ------------------------------------------------------------------------------------------
 * (4) Sparse shared-KV (MLA) attention with a per-head sink ([xLLM-CP] Design, data-flow
 * step (4): the local queries of all heads attend over the full KV stream's selected rows and
 * give [T_local, num_heads, head_dim]; key points: the attention sink is held for all heads).
 * For row i and head h over S = { idx[i, j] : idx[i, j] != -1 }:
 *   l_s = softmax_scale * q[i,h,:] . kv[s, :]
 *   out[i,h,:] = sum_s e^(l_s) kv[s, 0:d_v] / (e^(sink[h]) + sum_s e^(l_s))
 *   lse[i,h]   = ln(e^(sink[h]) + sum_s e^(l_s))
 * (no sink: sink == NULL drops the e^(sink) term). Accumulation is float32; out has q's dtype.
 * Supported: (n_heads, d_qk, d_v, dtype) = (128, 576, 512, bf16) with k_tot <= 2304 (matrix
 * cores), and float32 or bf16 with n_heads * d_v <= 4096, d_qk <= 512 and
 * n_heads * d_qk <= 16384 (vector ALU); anything else returns DSA_ERR_UNSUPPORTED. Row ids
 * outside [-1, n_rows) set DSA_DEVERR_INDEX in *err_flag and are skipped. A query with no
 * selected row gives out = 0 and lse = sink[h] (-inf without a sink).
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const void* q;            /* device [nq, n_heads, d_qk]                                    */
  const void* kv;           /* device [n_rows, d_qk]; value = columns [0, d_v)               */
  const int32_t* idx;       /* device [nq, k_tot] absolute row ids, -1 = none                */
  const float* sink;        /* device [n_heads] natural-log logits, or NULL                  */
  void* out;                /* device out [nq, n_heads, d_v], dtype `dtype`                  */
  float* lse;               /* device out [nq, n_heads] or NULL                              */
  int32_t* err_flag;        /* device [1] or NULL                                             */
  float softmax_scale;
  int32_t dtype;            /* dsa_dtype of q, kv and out (DSA_F32 or DSA_BF16)              */
  int32_t nq, n_rows, n_heads, d_qk, d_v, k_tot;
} dsa_sparse_attn_args;

dsa_status dsa_sparse_attn(const dsa_sparse_attn_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * (5) Rerange of a rank-concatenated buffer into logical token order ([CP-blog] Part 3 step B:
 * the all-gathered rows arrive as T0,T4, T1,T5, ... and are restored to T0,T1,T2,...;
 * [CP-gathers] Gather #1: the same helper undoes both the round-robin and the in-seq split).
 *   inverse = 0: out[t] = in[off(rank(t)) + local_row(t)] for t < num_tokens  (out: [T, row])
 *   inverse = 1: the split: out = rank-concatenated buffer of in (out: [num_rows_concat, row]),
 *                pad rows zero-filled.
 * Round-robin: rank(t) = t % cp, local_row(t) = t / cp; off(r) = r*tokens_per_rank when padded,
 * else the real rows of ranks < r. In-seq: the permutation is the identity (a copy).
 * row_bytes % 16 == 0; in and out must not overlap.
 * ------------------------------------------------------------------------------------------ */
dsa_status dsa_rerange(const void* in, void* out, int32_t num_tokens, int64_t row_bytes,
                       int32_t cp_size, int32_t mode, int32_t pad_to_cp, int32_t inverse,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
