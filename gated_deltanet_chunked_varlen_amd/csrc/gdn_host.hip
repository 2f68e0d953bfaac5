// gdn_host.hip -- the C ABI of libgdn_prefill: host-side checks, workspace
// planning and the launch sequence.
//
// Argument rules follow gitcode "FlashInfer GDN Prefill 完全指南" (sections
// "API 全参数解析", "状态池", "中间状态检查点", "约束与注意点"): head sharing
// (hq == hk and hv % hq == 0) or (hk == hv and hq % hk == 0); checkpoint
// interval a multiple of 64 with its two buffers given together; an output
// pool required with state_indices and a final state; max_seqlen within
// [ceil(T/N), T].  Nothing here reads device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/gdn_prefill.h"
#include "gdn_internal.h"

using namespace gdn;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int32_t sab_heads(const gdn_prefill_params *p) {
  return std::max(p->num_q_heads, p->num_v_heads);
}

size_t elem_size(int dtype) { return dtype == GDN_F32 ? 4 : 2; }

bool valid_state_dtype(int d) {
  return d == GDN_F32 || d == GDN_BF16 || d == GDN_F16 || d == GDN_FP8_E4M3 || d == GDN_FP8_E5M2;
}
bool valid_itype(int t) { return t == GDN_I32 || t == GDN_I64; }

// Context-parallel configuration of a call: segments of seg chunks, at most
// nseg per sequence (0, 0: the ordinary pass).  Decided from the parameter
// block alone (no device query: every gfx950 part has 256 compute units), so
// the workspace size is known before a device is touched.
constexpr int kCpCUs = 256;
constexpr int64_t kCpMinSegChunks = 16;
constexpr int64_t kCpMaxSegs = 4096;

bool cp_domain(const gdn_prefill_params *p) {
  return p->qkv_dtype != GDN_F32 && p->head_size == 128 && p->num_seqs >= 1 &&
         p->num_seqs <= kDirectSeqs && p->total_tokens > 0;
}

struct CpConfig {
  int32_t seg = 0, nseg = 0;
};

// Segment length: the batch's chunks over enough segments for two
// 16-column tiles per compute unit in the final pass (its two-tile form),
// and no shorter than kCpMinSegChunks chunks (the start-state fix-up is
// serial over a sequence's segments).  Measured on the MI355X with one to
// sixteen heads and 16 384 to 131 072 tokens per call: the best of segments
// of 1 024 ... 16 384 tokens sits at this choice or within 4 % of it.  Auto
// takes the context-parallel form when the ordinary pass occupies at most
// half of the compute units and the longest possible sequence spans two or
// more segments.
CpConfig cp_config(const gdn_prefill_params *p) {
  CpConfig c;
  if (p->use_cp == GDN_CP_OFF || !cp_domain(p)) return c;
  const int64_t maxlen = p->max_seqlen > 0 ? p->max_seqlen : p->total_tokens;
  const int64_t maxc = (maxlen + GDN_CHUNK - 1) / GDN_CHUNK;
  const int64_t H = std::max(p->num_q_heads, p->num_v_heads);
  const int64_t tiles = (int64_t)p->num_seqs * H * (p->head_size / 16);
  int64_t seg;
  if (p->cp_chunk_len > 0) {
    seg = p->cp_chunk_len / GDN_CHUNK;
  } else {
    const int64_t chunks = gdn_max_chunks(p->total_tokens, p->num_seqs);
    const int64_t target = 2 * kCpCUs;  // tiles of the final pass
    seg = std::max<int64_t>(kCpMinSegChunks, (chunks * H * (p->head_size / 16) + target - 1) / target);
  }
  seg = std::max<int64_t>(seg, 1);
  if (p->use_cp == GDN_CP_AUTO && (tiles > kCpCUs / 2 || maxc < 2 * seg)) return c;
  // bound the segment count (the grid), lengthening segments if needed
  if ((maxc + seg - 1) / seg > kCpMaxSegs) seg = (maxc + kCpMaxSegs - 1) / kCpMaxSegs;
  c.seg = (int32_t)std::min<int64_t>(seg, INT32_MAX);
  c.nseg = (int32_t)std::max<int64_t>(1, (maxc + seg - 1) / seg);
  return c;
}

struct Layout {
  size_t chunk_idx, chunk_tok, cu_chunks, seq_bos, n_chunks, Wf, Kf, Uf, Hf, Nf, Qf, Pf, Gw, Bw;
  size_t cp_start, cp_sloc, cp_m, total;
  bool fuse;
  CpConfig cp;
};

Layout plan(const gdn_prefill_params *p) {
  Layout L{};
  const int64_t cap = gdn_max_chunks(p->total_tokens, p->num_seqs);
  const int64_t H = sab_heads(p), D = p->head_size, N = p->num_seqs;
  const size_t es = elem_size(p->qkv_dtype);
  const size_t blocks = (size_t)cap * (size_t)H;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L.chunk_idx = take(sizeof(int32_t) * 2 * (size_t)std::max<int64_t>(cap, 1));
  L.chunk_tok = take(sizeof(int32_t) * 2 * (size_t)std::max<int64_t>(cap, 1));
  L.cu_chunks = take(sizeof(int32_t) * (size_t)(N + 1));
  L.seq_bos = take(sizeof(int32_t) * (size_t)(N + 1));
  L.n_chunks = take(sizeof(int32_t));
  // 16-bit inputs: the state pass forms the output itself and needs the q and
  // P fragments instead of chunk-start states and N in memory; the normalised
  // k and q fragments are kept once per k / q head (GQA / GVA share them)
  L.fuse = p->qkv_dtype != GDN_F32;
  const size_t kblocks = L.fuse ? (size_t)cap * p->num_k_heads : blocks;
  L.Wf = take(blocks * 64 * D * es);
  L.Kf = take(kblocks * 64 * D * es);
  L.Uf = take(blocks * 64 * D * es);
  if (L.fuse) {
    L.Qf = take((size_t)cap * p->num_q_heads * 64 * D * es);
    L.Pf = take(blocks * 64 * 64 * es);
  } else {
    L.Nf = take(blocks * 64 * D * es);
    L.Hf = take(blocks * D * D * es);
  }
  L.Gw = take(blocks * 64 * sizeof(float));
  // the T form's row scales (two rows of 64 floats per chunk-head)
  if (L.fuse) L.Bw = take(blocks * 128 * sizeof(float));
  L.cp = cp_config(p);
  if (L.cp.nseg > 0) {
    // fp32 [N][nseg][H][D][D] each: segment start states, and each segment's
    // state from a zero start and its transition matrix
    const size_t st = (size_t)N * L.cp.nseg * H * D * D * sizeof(float);
    L.cp_start = take(st);
    L.cp_sloc = take(st);
    L.cp_m = take(st);
  }
  L.total = off;
  return L;
}

bool strides_ok(const int64_t s[4], int64_t rows, int64_t H, int64_t D) {
  if (s[0] == 0 && s[1] == 0 && s[2] == 0 && s[3] == 0) return true;
  int64_t ext[4] = {rows, H, D, D};
  int idx[4] = {0, 1, 2, 3};
  for (int i = 0; i < 4; ++i)
    if (s[i] <= 0) return false;
  std::sort(idx, idx + 4, [&](int x, int y) { return s[x] < s[y]; });
  for (int k = 0; k + 1 < 4; ++k) {
    // a dimension of extent 1 never overlaps anything
    if (ext[idx[k]] <= 1) continue;
    if (s[idx[k + 1]] < s[idx[k]] * ext[idx[k]]) return false;
  }
  return true;
}

void fill_strides(const int64_t in[4], int64_t H, int64_t D, int64_t out[4]) {
  if (in[0] == 0 && in[1] == 0 && in[2] == 0 && in[3] == 0) {
    out[3] = 1;
    out[2] = D;
    out[1] = D * D;
    out[0] = H * D * D;
  } else {
    for (int i = 0; i < 4; ++i) out[i] = in[i];
  }
}

// q, k, v and output move in 16-byte vector accesses.
bool io_aligned(const gdn_prefill_params *p) {
  const void *ptrs[4] = {p->q, p->k, p->v, p->output};
  for (const void *x : ptrs)
    if ((uintptr_t)x % 16 != 0) return false;
  return true;
}

// Checks that the current device is a gfx950 and reports its CU count
// (cached per device).
int check_device(int *num_cus = nullptr) {
  static std::mutex mu;
  static int cached[64];
  static int cus[64];
  static bool init = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!init) {
    for (int i = 0; i < 64; ++i) cached[i] = cus[i] = 0;
    init = true;
  }
  if (dev < 0 || dev >= 64) return GDN_ERR_DEVICE;
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GDN_ERR_DEVICE;
    cached[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    cus[dev] = prop.multiProcessorCount;
  }
  if (num_cus) *num_cus = cus[dev];
  return cached[dev] == 1 ? GDN_OK : GDN_ERR_DEVICE;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(int code) {
  switch (code) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "a required pointer is NULL";
    case GDN_ERR_SHAPE: return "invalid token, sequence or head counts, or head size not in {32, 64, 128}";
    case GDN_ERR_HEAD_RATIO: return "illegal head sharing: need (hq == hk and hv % hq == 0) or (hk == hv and hq % hk == 0)";
    case GDN_ERR_DTYPE: return "unsupported dtype or index type";
    case GDN_ERR_CHECKPOINT: return "checkpoint_every_n_tokens must be a non-negative multiple of 64 and state_checkpoints / checkpoint_cu_starts must be given together";
    case GDN_ERR_STATE: return "inconsistent state arguments (output_state required for a final state; pool_size required with state_indices)";
    case GDN_ERR_MAX_SEQLEN: return "max_seqlen outside [ceil(total_tokens / num_seqs), total_tokens]";
    case GDN_ERR_WORKSPACE: return "workspace missing or smaller than gdn_prefill_workspace_size()";
    case GDN_ERR_STRIDES: return "state strides must be all zero (contiguous) or positive and non-overlapping";
    case GDN_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
    case GDN_ERR_LAUNCH: return "kernel launch failed";
    case GDN_ERR_ALIGN: return "q, k, v and output must be 16-byte aligned and the workspace 256-byte aligned";
    case GDN_ERR_CP: return "use_cp must be 0 (auto), 1 (on) or 2 (off) and cp_chunk_len a non-negative multiple of 64; use_cp = on needs bf16 or fp16 inputs, head size 128 and at most 63 sequences";
    case GDN_ERR_SCRATCH: return "gdn_prefill_noalloc: the call needs more workspace than the static scratch (GDN_NOALLOC_SCRATCH_BYTES) or its address is unavailable";
    case (int)GDN_STATUS_CU_SEQLENS: return "status: cu_seqlens not non-decreasing within [0, total_tokens]";
    case (int)GDN_STATUS_CHECKPOINT_STARTS: return "status: checkpoint_cu_starts differs from the prefix sum of floor(len / n)";
    case (int)GDN_STATUS_STATE_INDEX: return "status: a state index is outside [0, pool_size)";
    case (int)GDN_STATUS_CHUNK_CAPACITY: return "status: chunk table capacity exceeded";
    default: return "unknown code";
  }
}

int64_t gdn_max_chunks(int64_t total_tokens, int32_t num_seqs) {
  if (total_tokens <= 0 || num_seqs <= 0) return 0;
  const int64_t m = std::min<int64_t>(num_seqs, total_tokens);
  return (total_tokens + 63 * m) / 64;
}

static int check_shape(const gdn_prefill_params *p) {
  if (!p) return GDN_ERR_NULL;
  if (p->total_tokens < 0 || p->total_tokens > INT32_MAX - 64 || p->num_seqs < 0) return GDN_ERR_SHAPE;
  if (p->num_q_heads < 1 || p->num_k_heads < 1 || p->num_v_heads < 1) return GDN_ERR_SHAPE;
  if (p->head_size != 32 && p->head_size != 64 && p->head_size != 128) return GDN_ERR_SHAPE;
  if (!p->cu_seqlens && p->num_seqs != 1) return GDN_ERR_SHAPE;
  const int32_t hq = p->num_q_heads, hk = p->num_k_heads, hv = p->num_v_heads;
  const bool gva = (hq == hk) && (hv % hq == 0);
  const bool gqa = (hk == hv) && (hq % hk == 0);
  if (!gva && !gqa) return GDN_ERR_HEAD_RATIO;
  if (p->qkv_dtype != GDN_F32 && p->qkv_dtype != GDN_BF16 && p->qkv_dtype != GDN_F16)
    return GDN_ERR_DTYPE;
  return GDN_OK;
}

size_t gdn_prefill_workspace_size(const gdn_prefill_params *p) {
  if (check_shape(p) != GDN_OK) return 0;
  return plan(p).total;
}

int gdn_validate_host(const gdn_prefill_params *p) {
  int rc = check_shape(p);
  if (rc != GDN_OK) return rc;
  const int64_t T = p->total_tokens, N = p->num_seqs, H = sab_heads(p), D = p->head_size;
  if (T > 0 && (!p->q || !p->k || !p->v || !p->output)) return GDN_ERR_NULL;
  if (!io_aligned(p)) return GDN_ERR_ALIGN;
  if (p->cu_seqlens && !valid_itype(p->cu_seqlens_type)) return GDN_ERR_DTYPE;
  // states
  if (p->initial_state && !valid_state_dtype(p->initial_state_dtype)) return GDN_ERR_DTYPE;
  if (p->output_final_state) {
    if (!p->output_state) return GDN_ERR_STATE;
    if (!valid_state_dtype(p->output_state_dtype)) return GDN_ERR_DTYPE;
  }
  int64_t rows = N;
  if (p->state_indices) {
    if (!valid_itype(p->state_indices_type)) return GDN_ERR_DTYPE;
    if (p->pool_size < 1) return GDN_ERR_STATE;
    rows = p->pool_size;
  }
  if (p->initial_state && !strides_ok(p->initial_state_strides, rows, H, D)) return GDN_ERR_STRIDES;
  if (p->output_final_state && !strides_ok(p->output_state_strides, rows, H, D)) return GDN_ERR_STRIDES;
  // checkpoints
  if (p->checkpoint_every_n_tokens < 0) return GDN_ERR_CHECKPOINT;
  if ((p->state_checkpoints == nullptr) != (p->checkpoint_cu_starts == nullptr)) return GDN_ERR_CHECKPOINT;
  if (p->checkpoint_every_n_tokens > 0) {
    if (p->checkpoint_every_n_tokens % GDN_CHUNK != 0) return GDN_ERR_CHECKPOINT;
    if (!p->state_checkpoints) return GDN_ERR_CHECKPOINT;
    if (!valid_state_dtype(p->checkpoint_dtype)) return GDN_ERR_DTYPE;
    if (!valid_itype(p->checkpoint_cu_starts_type)) return GDN_ERR_DTYPE;
    if (p->checkpoint_rows < 0) return GDN_ERR_CHECKPOINT;
  }
  // max_seqlen
  if (p->max_seqlen < 0) return GDN_ERR_MAX_SEQLEN;
  if (p->max_seqlen > 0 && N > 0) {
    const int64_t lo = (T + N - 1) / N;
    if (p->max_seqlen < lo || p->max_seqlen > T) return GDN_ERR_MAX_SEQLEN;
  }
  // context parallelism
  if (p->use_cp < GDN_CP_AUTO || p->use_cp > GDN_CP_OFF) return GDN_ERR_CP;
  if (p->cp_chunk_len < 0 || p->cp_chunk_len % GDN_CHUNK != 0) return GDN_ERR_CP;
  if (p->use_cp == GDN_CP_ON && !cp_domain(p) && T > 0) return GDN_ERR_CP;
  // workspace
  const size_t need = plan(p).total;
  if (p->workspace_bytes < need || (need > 0 && !p->workspace)) return GDN_ERR_WORKSPACE;
  if ((uintptr_t)p->workspace % kAlign != 0) return GDN_ERR_ALIGN;
  return GDN_OK;
}

int gdn_build_chunk_indices(const void *cu_seqlens, int32_t cu_type, int32_t num_seqs,
                            int64_t total_tokens, int32_t *chunk_indices, int32_t *cu_chunks,
                            int32_t *seq_starts, int32_t *n_chunks, int32_t *status,
                            void *stream) {
  if (num_seqs < 0 || total_tokens < 0 || total_tokens > INT32_MAX - 64) return GDN_ERR_SHAPE;
  if (!cu_seqlens && num_seqs != 1) return GDN_ERR_SHAPE;
  if (cu_seqlens && !valid_itype(cu_type)) return GDN_ERR_DTYPE;
  const int64_t cap = gdn_max_chunks(total_tokens, num_seqs);
  if (!cu_chunks || !seq_starts || !n_chunks || (cap > 0 && !chunk_indices)) return GDN_ERR_NULL;
  int rc = check_device();
  if (rc != GDN_OK) return rc;
  hipError_t e = launch_chunk_index(cu_seqlens, cu_type, num_seqs, total_tokens, cap,
                                    chunk_indices, cu_chunks, seq_starts, n_chunks, status,
                                    nullptr, 0, 0, nullptr, 0, 0, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// The kernels' argument block for a call (workspace pointers only when a
// workspace layout is given).
// Above this many bytes of intermediates the fused pass finds them in HBM
// rather than in the 256 MB last-level cache (the intra-chunk pass streams
// q, k and v through it as well), and warming L2 ahead of the loads pays.
// Measured at 16 heads, D = 128 (intermediates over the chunk-count bound):
// plain stores and no warm-up are faster at 139 and 199 MB (7 and 10
// sequences of 1024 tokens), the large-call form at 229 and 260 MB (3 x 4096
// and 13 x 1024 tokens).
constexpr int64_t kWarmBytes = 200ll << 20;

static void fill_args(const gdn_prefill_params *p, const Layout *L, int num_cus, Args &a) {
  unsigned char *ws = (unsigned char *)p->workspace;
  const int64_t H = sab_heads(p), D = p->head_size;
  std::memset(&a, 0, sizeof(a));
  a.T = p->total_tokens;
  a.N = p->num_seqs;
  a.H = (int32_t)H;
  a.hq = p->num_q_heads;
  a.hk = p->num_k_heads;
  a.hv = p->num_v_heads;
  a.D = (int32_t)D;
  a.dtype = p->qkv_dtype;
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.g = p->g;
  a.beta = p->beta;
  a.scale = p->has_scale ? p->scale : (float)(1.0 / std::sqrt((double)D));
  a.l2norm = p->use_qk_l2norm_in_kernel ? 1 : 0;
  a.out = p->output;
  if (L) {
    a.chunk_idx = (int32_t *)(ws + L->chunk_idx);
    a.chunk_tok = (int32_t *)(ws + L->chunk_tok);
    a.cu_chunks = (int32_t *)(ws + L->cu_chunks);
    a.seq_bos = (int32_t *)(ws + L->seq_bos);
    a.n_chunks = (int32_t *)(ws + L->n_chunks);
    a.Wf = ws + L->Wf;
    a.Kf = ws + L->Kf;
    a.Uf = ws + L->Uf;
    if (L->fuse) {
      a.Qf = ws + L->Qf;
      a.Pf = ws + L->Pf;
      a.fuse = 1;
      // W, U (64 x D) and P (64 x 64) per chunk-head, K and q (64 x D) per
      // chunk and k / q head, 16-bit
      const int64_t inter = gdn_max_chunks(p->total_tokens, p->num_seqs) *
                            (H * (2 * 64 * D + 64 * 64) +
                             (int64_t)(p->num_k_heads + p->num_q_heads) * 64 * D) * 2;
      a.warm = inter > kWarmBytes ? 2 : 0;
      a.nt_stores = inter > kWarmBytes ? 1 : 0;
      // the state pass in its T form (16-bit D = 128 without context
      // parallelism) where its extra chain work pays: with two or four tiles
      // per workgroup (the CU's memory path bounds the step), or where the
      // intermediates would outgrow the last-level cache (the intra-chunk
      // pass's traffic halves).  Small one-tile calls are bound by the chain
      // and keep -W, Ktilde^T and U (2 x 2048 tokens x 16 heads: 52.7 us per
      // call against 60.6 in the T form; 262 144 tokens x 32 heads: 7.12 ms
      // against 6.42).
      const int64_t tiles = (int64_t)p->num_seqs * H * (D / 16);
      a.tform = (D == 128 && L->cp.nseg == 0 && (tiles > num_cus || inter > kWarmBytes)) ? 1 : 0;
    } else {
      a.Hf = ws + L->Hf;
      a.Nf = ws + L->Nf;
    }
    a.Gw = (float *)(ws + L->Gw);
    if (L->fuse) a.Bw = (float *)(ws + L->Bw);
    if (L->cp.nseg > 0) {
      a.cp_seg = L->cp.seg;
      a.cp_nseg = L->cp.nseg;
      a.cp_start = (float *)(ws + L->cp_start);
      a.cp_sloc = (float *)(ws + L->cp_sloc);
      a.cp_m = (float *)(ws + L->cp_m);
    }
  }
  a.cap = gdn_max_chunks(p->total_tokens, p->num_seqs);
  const int64_t rows = p->state_indices ? p->pool_size : p->num_seqs;
  a.init = p->initial_state;
  a.init_dtype = p->initial_state_dtype;
  fill_strides(p->initial_state_strides, H, D, a.init_str);
  a.init_rows = rows;
  a.outst = p->output_state;
  a.out_dtype = p->output_state_dtype;
  fill_strides(p->output_state_strides, H, D, a.out_str);
  a.out_final = p->output_final_state ? 1 : 0;
  a.sidx = p->state_indices;
  a.sidx_type = p->state_indices_type;
  a.pool_rows = rows;
  a.ck_every = p->checkpoint_every_n_tokens;
  a.ck = p->state_checkpoints;
  a.ck_dtype = p->checkpoint_dtype;
  const int64_t zero4[4] = {0, 0, 0, 0};
  fill_strides(zero4, H, D, a.ck_str);
  a.ck_rows = p->checkpoint_rows;
  a.ck_cs = p->checkpoint_cu_starts;
  a.ck_cs_type = p->checkpoint_cu_starts_type;
  a.status = p->status;
  a.num_cus = num_cus;
  a.cu = p->cu_seqlens;
  a.cu_type = p->cu_seqlens_type;
  // small batches: the kernels read the sequence geometry from cu_seqlens
  // themselves and the chunk-index builder is not launched
  a.direct = (a.N <= kDirectSeqs && a.cap > 0) ? 1 : 0;
  if (a.ck_every > 0 && !a.ck) a.ck_every = 0;
}

static int prefill_impl(const gdn_prefill_params *p, void *stream, void *const *events) {
  int rc = gdn_validate_host(p);
  if (rc != GDN_OK) return rc;
  int num_cus = 0;
  rc = check_device(&num_cus);
  if (rc != GDN_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const Layout L = plan(p);
  Args a;
  fill_args(p, &L, num_cus, a);

  auto mark = [&](int i) -> hipError_t {
    if (events && events[i]) return hipEventRecord((hipEvent_t)events[i], s);
    return hipSuccess;
  };
  hipError_t e = mark(0);
  if (e == hipSuccess && !a.direct)
    e = launch_chunk_index(p->cu_seqlens, p->cu_seqlens_type, a.N, a.T, a.cap, a.chunk_idx,
                           a.cu_chunks, a.seq_bos, a.n_chunks, a.status,
                           a.ck_every > 0 ? a.ck_cs : nullptr, a.ck_cs_type, a.ck_every,
                           a.sidx, a.sidx_type, a.pool_rows, a.chunk_tok, s);
  if (e == hipSuccess) e = mark(1);
  if (e == hipSuccess && a.cap > 0) e = launch_intra(a, s);
  if (e == hipSuccess) e = mark(2);
  if (a.fuse && a.cp_nseg > 0) {
    // context parallel: segment transitions, serial fix-up of the segment
    // start states, then the fused pass over every segment
    if (e == hipSuccess) e = launch_cp_transition(a, s);
    if (e == hipSuccess) e = launch_cp_fixup(a, s);
    if (e == hipSuccess) e = launch_state_output(a, s);
    if (e == hipSuccess) e = mark(3);
  } else if (a.fuse) {
    // state and output in one pass; the output phase is empty
    if (e == hipSuccess) e = launch_state_output(a, s);
    if (e == hipSuccess) e = mark(3);
  } else {
    if (e == hipSuccess) e = launch_state(a, s);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess && a.cap > 0) e = launch_output(a, s);
  }
  if (e == hipSuccess) e = mark(4);
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int gdn_prefill(const gdn_prefill_params *p, void *stream) {
  return prefill_impl(p, stream, nullptr);
}

// The no-allocation variant's workspace: one copy per GPU, created when the
// code object is loaded on that GPU.  In host code `scratch` is only a
// stand-in for the symbol; its device address comes from hipGetSymbolAddress,
// looked up once per device and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

static int scratch_address(void **out) {
  static std::mutex mu;
  static void *scratch_ptr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GDN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return GDN_ERR_SCRATCH;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return GDN_OK;
}

int gdn_prefill_noalloc(const gdn_prefill_params *p, void *stream) {
  if (!p) return GDN_ERR_NULL;
  gdn_prefill_params q = *p;
  q.workspace = nullptr;
  q.workspace_bytes = 0;
  const size_t need = gdn_prefill_workspace_size(&q);
  if (need == 0) {
    const int rc = gdn_validate_host(&q);
    return rc != GDN_OK ? rc : GDN_ERR_SHAPE;
  }
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
  int rc = check_device();
  if (rc != GDN_OK) return rc;
  rc = scratch_address(&q.workspace);
  if (rc != GDN_OK) return rc;
  q.workspace_bytes = GDN_NOALLOC_SCRATCH_BYTES;
  return prefill_impl(&q, stream, nullptr);
}

int gdn_validate_decode_host(const gdn_prefill_params *p) {
  if (!p) return GDN_ERR_NULL;
  if (p->num_seqs < 0 || p->total_tokens != p->num_seqs || p->cu_seqlens) return GDN_ERR_SHAPE;
  if (p->num_q_heads < 1 || p->num_k_heads < 1 || p->num_v_heads < 1) return GDN_ERR_SHAPE;
  if (p->head_size != 32 && p->head_size != 64 && p->head_size != 128) return GDN_ERR_SHAPE;
  const int32_t hq = p->num_q_heads, hk = p->num_k_heads, hv = p->num_v_heads;
  if (!((hq == hk && hv % hq == 0) || (hk == hv && hq % hk == 0))) return GDN_ERR_HEAD_RATIO;
  if (p->qkv_dtype != GDN_F32 && p->qkv_dtype != GDN_BF16 && p->qkv_dtype != GDN_F16)
    return GDN_ERR_DTYPE;
  if (p->checkpoint_every_n_tokens != 0 || p->state_checkpoints || p->checkpoint_cu_starts)
    return GDN_ERR_CHECKPOINT;
  const int64_t N = p->num_seqs, H = sab_heads(p), D = p->head_size;
  if (N > 0 && (!p->q || !p->k || !p->v || !p->output)) return GDN_ERR_NULL;
  if (!io_aligned(p)) return GDN_ERR_ALIGN;
  if (p->initial_state && !valid_state_dtype(p->initial_state_dtype)) return GDN_ERR_DTYPE;
  if (p->output_final_state) {
    if (!p->output_state) return GDN_ERR_STATE;
    if (!valid_state_dtype(p->output_state_dtype)) return GDN_ERR_DTYPE;
  }
  int64_t rows = N;
  if (p->state_indices) {
    if (!valid_itype(p->state_indices_type)) return GDN_ERR_DTYPE;
    if (p->pool_size < 1) return GDN_ERR_STATE;
    rows = p->pool_size;
  }
  if (p->initial_state && !strides_ok(p->initial_state_strides, rows, H, D)) return GDN_ERR_STRIDES;
  if (p->output_final_state && !strides_ok(p->output_state_strides, rows, H, D)) return GDN_ERR_STRIDES;
  return GDN_OK;
}

int gdn_decode(const gdn_prefill_params *p, void *stream) {
  int rc = gdn_validate_decode_host(p);
  if (rc != GDN_OK) return rc;
  int num_cus = 0;
  rc = check_device(&num_cus);
  if (rc != GDN_OK) return rc;
  Args a;
  fill_args(p, nullptr, num_cus, a);
  a.direct = 0;
  if (a.N == 0 && !a.status) return GDN_OK;
  const hipError_t e = launch_decode(a, (hipStream_t)stream);
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

int gdn_prefill_timed(const gdn_prefill_params *p, void *stream, void *const events[5]) {
  return prefill_impl(p, stream, events);
}

}  // extern "C"
