// k0_chunk_index.hip -- device-side chunk-index builder.
//
// weigao.cc "GDN 与 Chunked Prefill", sections "chunked prefill 有两层含义"
// and "为什么 trace 里它可能看起来很贵": the kernel chunks of a packed varlen
// batch are addressed through a flat table (flat chunk -> sequence, chunk
// within the sequence), sequence-major.  Built here on the device from
// cu_seqlens, so no length ever travels back to the host.
//
// One workgroup of 1024 threads:
//   pass 1  sanitised starts bos_i = running max of clamp(cu_i, 0, T)
//           (flags non-monotone or out-of-range cu_seqlens);
//   pass 2  n_i = ceil(len_i / 64), cu_chunks = exclusive scan; checkpoint
//           starts are recomputed and compared when given; state indices are
//           range-checked;
//   pass 3  every table slot f < cap: binary search of cu_chunks; beside the
//           (sequence, chunk) table, an optional (first token, length) table
//           that lets a chunk's workgroup find its rows with one load.
// Scans run tile by tile (1024 sequences per tile) with a carried prefix.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

constexpr int kK0Threads = 1024;
constexpr int kK0Lds = 4096;  // sequences whose starts / chunk offsets stay in LDS

__device__ __forceinline__ int64_t load_index(const void *p, int type, int64_t i) {
  return type == GDN_I64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

// Inclusive block scan (sum or max) over 1024 threads via wave scans + LDS.
template <bool kMax>
__device__ __forceinline__ int64_t block_scan(int64_t x, int64_t *sh_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int64_t y = __shfl_up(x, o);
    if (lane >= o) x = kMax ? (y > x ? y : x) : x + y;
  }
  if (lane == 63) sh_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int64_t w = lane < kK0Threads / 64 ? sh_wave[lane] : (kMax ? INT64_MIN : 0);
#pragma unroll
    for (int o = 1; o < kK0Threads / 64; o <<= 1) {
      int64_t y = __shfl_up(w, o);
      if (lane >= o) w = kMax ? (y > w ? y : w) : w + y;
    }
    if (lane < kK0Threads / 64) sh_wave[lane] = w;
  }
  __syncthreads();
  if (wave > 0) {
    int64_t pre = sh_wave[wave - 1];
    x = kMax ? (pre > x ? pre : x) : pre + x;
  }
  __syncthreads();
  return x;
}

__global__ void __launch_bounds__(kK0Threads)
chunk_index_kernel(const void *cu, int cu_type, int32_t N, int64_t T, int64_t cap,
                   int32_t *chunk_idx, int32_t *cu_chunks, int32_t *seq_bos,
                   int32_t *n_chunks, int32_t *status, const void *ck_cs,
                   int ck_cs_type, int32_t ck_every, const void *sidx,
                   int sidx_type, int64_t pool_rows, int32_t *chunk_tok) {
  __shared__ int64_t sh_wave[kK0Threads / 64];
  __shared__ int64_t sh_carry[2];
  __shared__ unsigned sh_status;
  __shared__ int32_t sh_bos[kK0Lds + 1], sh_cc[kK0Lds + 1];
  const bool small = N <= kK0Lds;
  const int tid = threadIdx.x;
  if (tid == 0) { sh_status = 0u; sh_carry[0] = 0; sh_carry[1] = 0; }
  __syncthreads();

  // pass 1: sanitised starts (running max of clamped offsets), i in [0, N].
  for (int64_t base = 0; base <= N; base += kK0Threads) {
    const int64_t i = base + tid;
    int64_t x = 0;
    if (i <= N) {
      int64_t raw = cu ? load_index(cu, cu_type, i) : (i == 0 ? 0 : T);
      x = raw < 0 ? 0 : (raw > T ? T : raw);
      bool bad = (raw != x);
      if (i > 0 && cu) bad |= raw < load_index(cu, cu_type, i - 1);
      if (bad) atomicOr(&sh_status, GDN_STATUS_CU_SEQLENS);
    }
    const int64_t carry = sh_carry[0];
    int64_t m = block_scan<true>(x, sh_wave);
    m = m > carry ? m : carry;
    if (i <= N) {
      seq_bos[i] = (int32_t)m;
      if (small) sh_bos[i] = (int32_t)m;
    }
    if (tid == kK0Threads - 1) sh_carry[0] = m;
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();

  // pass 2: chunk counts, exclusive scan; checkpoint starts; state indices.
  sh_carry[0] = 0;
  __syncthreads();
  for (int64_t base = 0; base <= N; base += kK0Threads) {
    const int64_t i = base + tid;
    int64_t nch = 0, nck = 0;
    if (i < N) {
      const int64_t len = small ? (int64_t)sh_bos[i + 1] - sh_bos[i]
                                : (int64_t)seq_bos[i + 1] - seq_bos[i];
      nch = (len + kChunk - 1) / kChunk;
      nck = ck_every > 0 ? len / ck_every : 0;
      if (sidx) {
        const int64_t r = load_index(sidx, sidx_type, i);
        if (r < 0 || r >= pool_rows) atomicOr(&sh_status, GDN_STATUS_STATE_INDEX);
      }
    }
    const int64_t c0 = sh_carry[0], c1 = sh_carry[1];
    const int64_t inc_c = block_scan<false>(nch, sh_wave);
    const int64_t inc_k = block_scan<false>(nck, sh_wave);
    if (i <= N) {
      const int64_t ex_c = c0 + inc_c - nch;
      cu_chunks[i] = (int32_t)ex_c;
      if (small) sh_cc[i] = (int32_t)ex_c;
      if (ck_cs && ck_every > 0) {
        const int64_t ex_k = c1 + inc_k - nck;
        if (load_index(ck_cs, ck_cs_type, i) != ex_k)
          atomicOr(&sh_status, GDN_STATUS_CHECKPOINT_STARTS);
      }
    }
    if (tid == kK0Threads - 1) { sh_carry[0] = c0 + inc_c; sh_carry[1] = c1 + inc_k; }
    __syncthreads();
  }
  __threadfence_block();
  __syncthreads();

  const int32_t *cc = small ? sh_cc : cu_chunks;
  int64_t total = cc[N];
  if (total > cap) {
    if (tid == 0) atomicOr(&sh_status, GDN_STATUS_CHUNK_CAPACITY);
    total = cap;
  }
  // pass 3: table entries
  for (int64_t f = tid; f < cap; f += kK0Threads) {
    int32_t si = -1, sc = -1, tb = 0, tl = 0;
    if (f < total) {
      int lo = 0, hi = N - 1;  // largest i in [0, N-1] with cu_chunks[i] <= f
      while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (cc[mid] <= f) lo = mid; else hi = mid - 1;
      }
      si = lo;
      sc = (int32_t)(f - cc[lo]);
      const int32_t b0 = small ? sh_bos[lo] : seq_bos[lo];
      const int32_t b1 = small ? sh_bos[lo + 1] : seq_bos[lo + 1];
      tb = b0 + kChunk * sc;
      tl = min(kChunk, b1 - tb);
    }
    chunk_idx[2 * f] = si;
    chunk_idx[2 * f + 1] = sc;
    if (chunk_tok) {
      chunk_tok[2 * f] = tb;
      chunk_tok[2 * f + 1] = tl;
    }
  }
  __syncthreads();
  if (tid == 0) {
    n_chunks[0] = (int32_t)total;
    if (status) status[0] = (int32_t)sh_status;
  }
}

hipError_t launch_chunk_index(const void *cu, int cu_type, int32_t N, int64_t T,
                              int64_t cap, int32_t *chunk_idx, int32_t *cu_chunks,
                              int32_t *seq_bos, int32_t *n_chunks, int32_t *status,
                              const void *ck_cs, int ck_cs_type, int32_t ck_every,
                              const void *sidx, int sidx_type, int64_t pool_rows,
                              int32_t *chunk_tok, hipStream_t s) {
  hipLaunchKernelGGL(chunk_index_kernel, dim3(1), dim3(kK0Threads), 0, s, cu, cu_type,
                     N, T, cap, chunk_idx, cu_chunks, seq_bos, n_chunks, status, ck_cs,
                     ck_cs_type, ck_every, sidx, sidx_type, pool_rows, chunk_tok);
  return hipGetLastError();
}

}  // namespace gdn
