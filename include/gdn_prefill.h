/*
 * gdn_prefill.h -- C ABI of libgdn_prefill: the varlen chunked Gated Delta
 * Rule prefill scan on AMD MI355X (gfx950).
 *
 * What is computed (gitcode "FlashInfer GDN Prefill 完全指南", sections
 * "GDN prefill" and "API 全参数解析"; weigao.cc "GDN 与 Chunked Prefill",
 * sections "GDN 是什么" and "块内 state 和块间 final state"): for every
 * sequence i of a packed varlen batch and every sab head h,
 *
 *     S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * with S a head_size x head_size fp32 state (keys x values) that starts from
 * the given initial state (or zero), is processed in 64-token chunks, and
 * whose final value is optionally written out.  g is alpha itself (the forget
 * gate, default all ones), beta the update gate (default all ones), scale
 * defaults to 1/sqrt(head_size).
 *
 * Conventions shared by every entry point:
 *  - Device pointers unless a comment says "host".  The caller owns every
 *    buffer; the library never allocates, frees or synchronises.  All work is
 *    enqueued on `stream` (a hipStream_t; NULL = the default stream) and the
 *    call returns without waiting.  No device-to-host copy happens in a call.
 *  - Return value: 0 on success, a negative GDN_ERR_* code when a host-side
 *    check fails (then nothing is launched).  gdn_status_string() names codes.
 *  - Data that only the device can check (cu_seqlens contents, state_indices
 *    values, checkpoint_cu_starts contents) never causes an out-of-bounds
 *    access; violations set GDN_STATUS_* bits in the optional device word
 *    `status`, which every call overwrites (it needs no clearing).
 */
#ifndef GDN_PREFILL_H
#define GDN_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2
#define GDN_CHUNK 64 /* kernel chunk length in tokens */

/* Element types.  The two 8-bit float types (OCP FP8 E4M3, max 448, and
 * E5M2, max 57344) are for states only -- initial, final and checkpoint
 * states (gitcode, section "chunk_gated_delta_rule API 全参数解析" lists them
 * for initial_state, section "中间状态检查点" for state_checkpoints).  The
 * pages give no scaling rule for them, so a state is stored by rounding each
 * fp32 element to nearest (ties to even) with saturation at the largest
 * finite value, and read by exact widening. */
typedef enum {
  GDN_F32 = 0, GDN_BF16 = 1, GDN_F16 = 2, GDN_FP8_E4M3 = 3, GDN_FP8_E5M2 = 4
} gdn_dtype;
typedef enum { GDN_I32 = 0, GDN_I64 = 1 } gdn_itype;

/* Host-side error codes (return values). */
#define GDN_OK 0
#define GDN_ERR_NULL -1          /* a required pointer is NULL */
#define GDN_ERR_SHAPE -2         /* token/sequence/head counts or head size */
#define GDN_ERR_HEAD_RATIO -3    /* illegal q/k/v head sharing */
#define GDN_ERR_DTYPE -4         /* unsupported dtype or index type */
#define GDN_ERR_CHECKPOINT -5    /* checkpoint arguments inconsistent */
#define GDN_ERR_STATE -6         /* state / pool arguments inconsistent */
#define GDN_ERR_MAX_SEQLEN -7    /* max_seqlen outside [ceil(T/N), T] */
#define GDN_ERR_WORKSPACE -8     /* workspace missing or too small */
#define GDN_ERR_STRIDES -9       /* state strides not positive/non-overlapping */
#define GDN_ERR_DEVICE -10       /* current device is not gfx950 */
#define GDN_ERR_LAUNCH -11       /* a kernel launch failed */
#define GDN_ERR_ALIGN -12        /* q, k, v or output not 16-byte aligned, or the
                                    workspace not 256-byte aligned (the kernels
                                    move them in 16-byte vector accesses) */
#define GDN_ERR_CP -14          /* use_cp outside {0, 1, 2}, cp_chunk_len not a
                                    non-negative multiple of 64, or GDN_CP_ON
                                    for a call outside the CP domain */
#define GDN_ERR_SCRATCH -13      /* gdn_prefill_noalloc(): the call needs more
                                    workspace than GDN_NOALLOC_SCRATCH_BYTES, or
                                    the static scratch's address is unavailable */

/* Size of the static device scratch that gdn_prefill_noalloc() uses in place
 * of a workspace (one copy per GPU, held until the process ends). */
#define GDN_NOALLOC_SCRATCH_BYTES (128u << 20)

/* Device status bits (written to *status by every call). */
#define GDN_STATUS_CU_SEQLENS 1u        /* cu_seqlens not non-decreasing within [0, T] */
#define GDN_STATUS_CHECKPOINT_STARTS 2u /* checkpoint_cu_starts != prefix sum of floor(len/n) */
#define GDN_STATUS_STATE_INDEX 4u       /* a state index outside [0, pool_size) */
#define GDN_STATUS_CHUNK_CAPACITY 8u    /* more chunks than the sync-free bound (never expected) */

/*
 * Parameters of one prefill call (gitcode, section "API 全参数解析"; the
 * fields keep that section's parameter names).
 *
 * Shapes, all row-major and contiguous unless strides are given:
 *   q [T, num_q_heads, D], k [T, num_k_heads, D], v [T, num_v_heads, D],
 *   qkv_dtype F32, BF16 or F16 (gitcode, section "覆盖的公共输入域", names
 *   FP16 and BF16 inputs).  Intermediates are kept in the input type for BF16
 *   and F16 and in fp32 for F32; accumulation is always fp32.
 *   H = num_sab_heads = max(num_q_heads, num_v_heads); legal head sharing:
 *   (hq == hk and hv % hq == 0) or (hk == hv and hq % hk == 0); sab head h
 *   reads q head h / (H / hq), k head h / (H / hk), v head h / (H / hv).
 *   g, beta [T, H] fp32, or NULL for all ones.  g is alpha in (0, 1].
 *   output [T, H, D] in qkv_dtype; rows outside every sequence are untouched.
 *   States are [rows, H, D(v), D(k)]: element [n][h][v][k] is S[k][v]; the
 *   four element strides are given (all zero = contiguous).  initial_state
 *   may be NULL (zero).  state dtypes: F32, BF16, F16, FP8_E4M3 or FP8_E5M2.
 *   state_indices [N] (or NULL): sequence i reads initial_state[idx[i]] and,
 *   if output_final_state, writes output_state[idx[i]]; indices must be
 *   unique (caller precondition, gitcode section "状态池"); output_state may
 *   be the same memory as initial_state (in-place pool); pool_size bounds the
 *   indices and is the row count of both pools.  Without state_indices,
 *   initial_state and output_state have N rows.
 *   checkpoint_every_n_tokens: 0 = off, else a positive multiple of 64;
 *   state_checkpoints [checkpoint_rows, H, D, D] (contiguous; rows outside
 *   [0, checkpoint_rows) are never written) and checkpoint_cu_starts
 *   [N+1] are then both required; checkpoint j (1-based) of sequence i is the
 *   state after j*n of its tokens, at row checkpoint_cu_starts[i] + j - 1.
 *   max_seqlen: 0 = unknown; otherwise must satisfy ceil(T/N) <= max_seqlen
 *   <= T (gitcode section "约束与注意点").
 *   Alignment: q, k, v and output start on 16-byte boundaries and the
 *   workspace on a 256-byte boundary (GDN_ERR_ALIGN otherwise; torch
 *   allocations satisfy both).
 */
typedef struct gdn_prefill_params {
  int64_t total_tokens;   /* T >= 0 */
  int32_t num_seqs;       /* N >= 0; with cu_seqlens NULL, N must be 1 */
  int32_t num_q_heads, num_k_heads, num_v_heads;
  int32_t head_size;      /* D in {32, 64, 128} */
  int32_t qkv_dtype;      /* gdn_dtype */
  const void *q, *k, *v;
  const float *g, *beta;
  int32_t has_scale;
  float scale;
  const void *cu_seqlens; /* [N+1], NULL = one sequence [0, T] */
  int32_t cu_seqlens_type; /* gdn_itype */
  int32_t use_qk_l2norm_in_kernel; /* x / sqrt(sum x^2 + 1e-6), fp32 sums */
  void *output;
  const void *initial_state;
  int32_t initial_state_dtype;
  int64_t initial_state_strides[4];
  int32_t output_final_state;
  void *output_state;
  int32_t output_state_dtype;
  int64_t output_state_strides[4];
  const void *state_indices;
  int32_t state_indices_type;
  int64_t pool_size;
  int32_t checkpoint_every_n_tokens;
  void *state_checkpoints;
  int32_t checkpoint_dtype;
  int64_t checkpoint_rows;
  const void *checkpoint_cu_starts;
  int32_t checkpoint_cu_starts_type;
  int64_t max_seqlen;
  void *workspace;
  size_t workspace_bytes;
  int32_t *status;        /* optional device word */
  /* Context parallelism within the GPU (gitcode, sections "API 全参数解析"
   * (use_cp, _cp_chunk_len, max_seqlen) and "Cake GDN CP 后端" ("四阶段执行
   * 流程"): each sequence is cut into segments of cp_chunk_len tokens, each
   * segment's state transition is formed in parallel, the segment start
   * states are fixed up serially, then every segment runs the ordinary pass
   * from its start state.  use_cp: GDN_CP_AUTO (0) takes it when the call has
   * too few (sequence, head) pairs to fill the GPU and long sequences;
   * GDN_CP_ON (1) requires it and fails closed (GDN_ERR_CP) outside its
   * domain (bf16 / fp16 inputs, head size 128, at most 63 sequences);
   * GDN_CP_OFF (2) never takes it.  cp_chunk_len: 0 = chosen from the shape
   * and max_seqlen (or total_tokens), else a positive multiple of 64 (for
   * tests and tuning).  The results are those of the non-CP pass up to
   * floating-point rounding. */
  int32_t use_cp;
  int64_t cp_chunk_len;
} gdn_prefill_params;

#define GDN_CP_AUTO 0
#define GDN_CP_ON 1
#define GDN_CP_OFF 2

/* ABI version (GDN_ABI_VERSION). */
int gdn_abi_version(void);

/* Static text for an error code (negative) or a status bit (positive). */
const char *gdn_status_string(int code);

/* Upper bound on the number of 64-token chunks of any batch with T tokens
 * and N sequences, needing no look at cu_seqlens:
 * floor((T + 63 * min(N, T)) / 64).  Host only. */
int64_t gdn_max_chunks(int64_t total_tokens, int32_t num_seqs);

/* Bytes of device workspace gdn_prefill() needs for these parameters (only
 * the shape fields are read: token, sequence and head counts, head size,
 * qkv dtype).  The pages' call allocates its scratch internally (gitcode,
 * section "内部机制：plan 缓存、地址重绑定与 CUDA Graph": a cached plan
 * holds the scratch of a shape); here the caller owns it, sized by this
 * function, so a call never allocates.  Host only; 0 for an invalid shape. */
size_t gdn_prefill_workspace_size(const gdn_prefill_params *p);

/* Every host-side check of gdn_prefill() except the device check, without
 * touching the GPU: the argument rules of gitcode, sections "API 全参数解析"
 * (shapes, dtypes, head sharing, defaults), "状态池" (state_indices needs
 * output_state and pool_size), "中间状态检查点" (n a multiple of 64, the two
 * checkpoint buffers given together) and "约束与注意点" (max_seqlen within
 * [ceil(T/N), T]), plus the workspace size and alignment.  Reads only the
 * parameter block, never device memory.  Returns GDN_OK or the GDN_ERR_*
 * code of the first failed check. */
int gdn_validate_host(const gdn_prefill_params *p);

/* The whole prefill (gitcode, sections "GDN prefill" and "API 全参数解析";
 * weigao.cc, "为什么要切成 64-token chunk"): the chunk-index build (large
 * batches only), the intra-chunk pass (gate log-cumsum, A, T), and the fused
 * pass that carries each state across chunks, writes checkpoints and the
 * final state (pool row state_indices[i] when given), and forms the output.
 * Runs gdn_validate_host() first and launches nothing when it fails.
 * Asynchronous on `stream`; returns GDN_OK once everything is enqueued, or
 * GDN_ERR_DEVICE (not a gfx950) / GDN_ERR_LAUNCH.  Data errors only the
 * device can see set bits in *status. */
int gdn_prefill(const gdn_prefill_params *p, void *stream);

/* gdn_prefill() with phase markers: events[i] (a hipEvent_t, or NULL to
 * skip) is recorded on `stream` just before phase i -- 0 chunk-index build,
 * 1 intra-chunk pass, 2 state pass, 3 output pass -- and events[4] after the
 * last, so hipEventElapsedTime(events[i], events[i + 1]) times phase i.  The
 * computation is exactly that of gdn_prefill().  events is a host array. */
int gdn_prefill_timed(const gdn_prefill_params *p, void *stream,
                      void *const events[5]);

/* gdn_prefill() for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a file-scope static device array of GDN_NOALLOC_SCRATCH_BYTES
 * (128 MiB) instead of p->workspace / p->workspace_bytes, which are ignored.
 * The caller still passes every input and output.  Nothing is allocated: no
 * hipMalloc, no hipFree, no allocating library call.  The first call on a
 * device looks up that device's copy of the array (hipGetSymbolAddress) and
 * keeps its address.  Returns GDN_ERR_SCRATCH when
 * gdn_prefill_workspace_size(p) exceeds GDN_NOALLOC_SCRATCH_BYTES (nothing
 * is launched), otherwise exactly what gdn_prefill() returns, with the same
 * results.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind; no part of it needs to start at zero (every call writes
 * what it reads), but calls that overlap in time on one GPU (different
 * streams, or different host threads without ordering) race on it. */
int gdn_prefill_noalloc(const gdn_prefill_params *p, void *stream);

/*
 * One decode step: one new token per sequence, applied to the state with the
 * recurrence itself, no chunking (weigao.cc "GDN 与 Chunked Prefill", section
 * "Prefill 和 decode 的差异": after prefill each step adds a single token,
 * S <- alpha (I - beta k k^T) S + beta k v^T and o = scale * S^T q with the
 * updated S; gitcode "FlashInfer GDN Prefill 完全指南", sections "GDN
 * prefill" and "状态池": decode continues from the state prefill leaves, in
 * the same [rows, H, V, K] layout and state_indices pool).
 *
 * Takes the prefill parameter block with these differences:
 *   - token i is the new token of sequence i: total_tokens == num_seqs, and
 *     cu_seqlens must be NULL (GDN_ERR_SHAPE otherwise); q/k/v are
 *     [N, heads, D], g and beta [N, H], output [N, H, D];
 *   - checkpoint_every_n_tokens must be 0 and the checkpoint buffers NULL
 *     (GDN_ERR_CHECKPOINT); max_seqlen and the workspace are ignored;
 *   - q, k, v and output 16-byte aligned as in gdn_prefill (GDN_ERR_ALIGN);
 *     states whose rows are not 16-byte aligned are read and written element
 *     by element.
 * States, pools (output_state may alias initial_state), head sharing,
 * defaults, l2 normalisation and the status word behave as in gdn_prefill;
 * only GDN_STATUS_STATE_INDEX can be set.  Duplicate state_indices race.
 */
int gdn_decode(const gdn_prefill_params *p, void *stream);

/* The host-side checks of gdn_decode() alone; no GPU needed. */
int gdn_validate_decode_host(const gdn_prefill_params *p);

/*
 * The device-side chunk-index builder alone (weigao.cc, sections "chunked
 * prefill 有两层含义" and "为什么 trace 里它可能看起来很贵": the flat chunk ->
 * (sequence, chunk) table built on the device, with no device-to-host copy).
 *   cu_seqlens [N+1] (int32 or int64 per cu_type).
 *   chunk_indices [cap][2] int32: entry f = (sequence, chunk in sequence),
 *     sequence-major; entries at f >= n_chunks are (-1, -1).
 *     cap = gdn_max_chunks(total_tokens, num_seqs).
 *   cu_chunks [N+1] int32: exclusive prefix sum of ceil(len_i / 64).
 *   seq_starts [N+1] int32: the sequence starts actually used: cu_seqlens
 *     clamped into [0, T] and made non-decreasing (running maximum), so the
 *     table never exceeds cap even for invalid input (which also sets
 *     GDN_STATUS_CU_SEQLENS in *status).  Equal to cu_seqlens when it is
 *     valid.
 *   n_chunks [1] int32.  status: optional device word.
 * Every output buffer is caller-owned; cu_seqlens NULL means one sequence
 * [0, T] (num_seqs must then be 1).
 */
int gdn_build_chunk_indices(const void *cu_seqlens, int32_t cu_type,
                            int32_t num_seqs, int64_t total_tokens,
                            int32_t *chunk_indices, int32_t *cu_chunks,
                            int32_t *seq_starts, int32_t *n_chunks,
                            int32_t *status, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_PREFILL_H */
