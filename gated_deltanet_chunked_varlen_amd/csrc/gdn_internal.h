// gdn_internal.h -- argument block and launchers of the GDN prefill kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/gdn_prefill.h"
#include "gdn_common.h"

namespace gdn {

// Largest batch whose sequence geometry one wave64 holds (lane i = sequence i,
// lane N = the end offset).
constexpr int kDirectSeqs = 63;

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (the attribute belongs to the device current when it is set);
// `done` holds one bit per device id below 64.  Threads that race both set
// it, which is harmless.
inline hipError_t set_dynamic_lds(const void *fn, int bytes, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Everything a kernel may read, passed by value.  Pointers are device
// pointers; strides are in elements.
struct Args {
  int64_t T;
  int32_t N, H, hq, hk, hv, D;
  int32_t dtype;  // 0 fp32, 1 bf16
  const void *q, *k, *v;
  const float *g, *beta;
  float scale;
  int32_t l2norm;
  void *out;
  // cu_seqlens (NULL: one sequence [0, T]); with direct != 0 the kernels
  // derive sequence and chunk geometry from it themselves (N <= kDirectSeqs)
  // and the tables below are not built
  const void *cu;
  int32_t cu_type;
  int32_t direct;
  // chunk table (written by the chunk-index builder)
  int32_t *chunk_idx;  // [cap][2]
  int32_t *cu_chunks;  // [N+1]
  int32_t *seq_bos;    // [N+1] sanitised sequence starts
  int32_t *n_chunks;   // [1]
  int32_t *chunk_tok;  // [cap][2] first token, length (0 for unused slots)
  int64_t cap;
  // intermediates
  void *Wf, *Kf, *Uf, *Hf, *Nf;
  // operands of the output products when the state pass produces the output
  // itself (fuse != 0): normalised q and masked Q K^T as fragments
  void *Qf, *Pf;
  int32_t fuse;
  float *Gw;
  // T form of the four-tile fused pass (tform != 0, set by the host when the
  // state pass takes that form): Wf holds -T diag(beta exp(G)) per chunk-head
  // as 64 x 64 operand fragments instead of -W, Kf is not written, and Bw
  // holds per chunk-head two rows of 64 floats: 1 / |k_t| and
  // exp(G_last - G_t) / |k_t| (0 past the chunk's end); the state pass reads
  // the raw k rows from the input
  float *Bw;
  int32_t tform;
  // states
  const void *init;
  int32_t init_dtype;
  int64_t init_str[4];
  int64_t init_rows;
  void *outst;
  int32_t out_dtype;
  int64_t out_str[4];
  int32_t out_final;
  const void *sidx;
  int32_t sidx_type;
  // checkpoints
  int32_t ck_every;
  void *ck;
  int32_t ck_dtype;
  int64_t ck_str[4];
  int64_t ck_rows;
  const void *ck_cs;
  int32_t ck_cs_type;
  // validation
  int64_t pool_rows;  // rows addressable through state_indices
  int32_t *status;
  int32_t num_cus;    // compute units of the device (launch shapes)
  // fused 16-bit pass: chunks ahead of the current step whose operand lines
  // one wave pulls into L2 (0: off; set when the intermediates outgrow the
  // last-level cache and the pass would read them from HBM)
  int32_t warm;
  // context parallelism (16-bit inputs, direct mode): each sequence splits
  // into segments of cp_seg chunks, at most cp_nseg of them; fp32
  // [N][cp_nseg][H][D][D] buffers hold each segment's start state, its state
  // from a zero start and its transition (row m = the transition's column m)
  int32_t cp_seg, cp_nseg;
  float *cp_start, *cp_sloc, *cp_m;
  // 16-bit intra-chunk pass, set with warm: write the intermediates with
  // non-temporal stores.  They then outgrow the last-level cache and are read
  // back from HBM anyway; below that size plain stores leave them in the
  // last-level cache for the state pass.
  int32_t nt_stores;
};

#ifdef __HIPCC__
// Data checks of a small batch (direct mode), by one wave: the chunk-index
// builder's checks on cu_seqlens, checkpoint_cu_starts and state_indices,
// written to *status as one word.
__device__ __forceinline__ void validate_direct(const Args &a, const SeqLane &s, int lane) {
  const int N = a.N;
  unsigned bits = 0;
  const long long prev = __shfl_up((long long)s.raw, 1);
  if (a.cu && lane <= N) {
    if (s.raw < 0 || s.raw > a.T || (lane > 0 && s.raw < prev)) bits |= GDN_STATUS_CU_SEQLENS;
  }
  if (a.ck_cs && a.ck_every > 0) {
    const int nck = lane < N ? s.len / a.ck_every : 0;
    int inc = nck;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o);
      if (lane >= o) inc += y;
    }
    if (lane <= N && load_index_any(a.ck_cs, a.ck_cs_type, lane) != (int64_t)(inc - nck))
      bits |= GDN_STATUS_CHECKPOINT_STARTS;
  }
  if (a.sidx && lane < N) {
    const int64_t r = load_index_any(a.sidx, a.sidx_type, lane);
    if (r < 0 || r >= a.pool_rows) bits |= GDN_STATUS_STATE_INDEX;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) bits |= __shfl_xor(bits, o);
  if (lane == 0) a.status[0] = (int32_t)bits;
}

// (first token, length) of flat chunk f for the calling wave: from the chunk
// table, or in direct mode from cu_seqlens (length 0: no such chunk).  With
// validate, the wave also runs the data checks of direct mode.
__device__ __forceinline__ void chunk_geometry(const Args &a, int f, int lane, bool validate,
                                               int &tok, int &len) {
  if (a.direct) {
    const SeqLane s = seq_lane(a.cu, a.cu_type, a.N, a.T, lane);
    if (validate && a.status) validate_direct(a, s, lane);
    chunk_from_lanes(s, a.N, f, lane, tok, len);
  } else {
    tok = a.chunk_tok[2 * f];
    len = a.chunk_tok[2 * f + 1];
  }
}

// Workspace blocks of the normalised k and q fragments for 16-bit inputs: one
// per (chunk, k head) and (chunk, q head), shared by every sab head that reads
// that k or q head (GQA / GVA), at index src_head * cap + f.  ch is the sab
// head's block index h * cap + f.
__device__ __forceinline__ int64_t k_block(const Args &a, int64_t ch, int h) {
  return ch + ((int64_t)(h / (a.H / a.hk)) - h) * a.cap;
}
__device__ __forceinline__ int64_t q_block(const Args &a, int64_t ch, int h) {
  return ch + ((int64_t)(h / (a.H / a.hq)) - h) * a.cap;
}

// First flat chunk, chunk count, length and first token of sequence seq, for
// the calling wave.
__device__ __forceinline__ void seq_geometry(const Args &a, int seq, int lane, int &f0, int &nc,
                                             int &len, int &bos) {
  if (a.direct) {
    const SeqLane s = seq_lane(a.cu, a.cu_type, a.N, a.T, lane);
    f0 = __shfl(s.cc0, seq);
    nc = __shfl(s.cc1, seq) - f0;
    len = __shfl(s.len, seq);
    bos = __shfl(s.bos, seq);
  } else {
    f0 = a.cu_chunks[seq];
    nc = min(a.cu_chunks[seq + 1], a.n_chunks[0]) - f0;
    len = a.seq_bos[seq + 1] - a.seq_bos[seq];
    bos = a.seq_bos[seq];
  }
}

__device__ __forceinline__ void seq_geometry(const Args &a, int seq, int lane, int &f0, int &nc,
                                             int &len) {
  int bos;
  seq_geometry(a, seq, lane, f0, nc, len, bos);
}

// The sequence of rank r when sequences are ordered by decreasing chunk
// count (ties by index), from the lanes' geometry s of a direct-mode batch.
// Workgroups taken in this order start the longest chains first, so a batch
// of uneven lengths that needs several rounds of workgroups does not end on
// a tail of its longest chains.
__device__ __forceinline__ int seq_by_length(const SeqLane &s, int N, int r, int lane) {
  const int n = lane < N ? s.cc1 - s.cc0 : -1;
  int rank = 0;
  for (int j = 0; j < N; ++j) {
    const int nj = __shfl(n, j);
    rank += (nj > n || (nj == n && j < lane)) ? 1 : 0;
  }
  const unsigned long long m = __ballot(lane < N && rank == r);
  return m ? __ffsll((long long)m) - 1 : r;
}

// seq_geometry for the workgroup of unit rank r, longest sequences first in
// direct mode (cu_seqlens read once for both); batch order with the chunk
// table.
__device__ __forceinline__ int seq_geometry_by_length(const Args &a, int r, int lane, int &f0,
                                                      int &nc, int &len, int &bos) {
  if (a.direct) {
    const SeqLane s = seq_lane(a.cu, a.cu_type, a.N, a.T, lane);
    const int seq = seq_by_length(s, a.N, r, lane);
    f0 = __shfl(s.cc0, seq);
    nc = __shfl(s.cc1, seq) - f0;
    len = __shfl(s.len, seq);
    bos = __shfl(s.bos, seq);
    return seq;
  }
  seq_geometry(a, r, lane, f0, nc, len, bos);
  return r;
}
#endif

// Chunk-index builder: one workgroup.
hipError_t launch_chunk_index(const void *cu, int cu_type, int32_t N, int64_t T,
                              int64_t cap, int32_t *chunk_idx, int32_t *cu_chunks,
                              int32_t *seq_bos, int32_t *n_chunks, int32_t *status,
                              const void *ck_cs, int ck_cs_type, int32_t ck_every,
                              const void *sidx, int sidx_type, int64_t pool_rows,
                              int32_t *chunk_tok, hipStream_t s);
hipError_t launch_intra(const Args &a, hipStream_t s);
hipError_t launch_state(const Args &a, hipStream_t s);
hipError_t launch_output(const Args &a, hipStream_t s);
hipError_t launch_decode(const Args &a, hipStream_t s);
hipError_t launch_state_output(const Args &a, hipStream_t s);
hipError_t launch_cp_transition(const Args &a, hipStream_t s);
hipError_t launch_cp_fixup(const Args &a, hipStream_t s);

}  // namespace gdn
