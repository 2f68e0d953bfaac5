// gdn_internal.h -- argument block and launchers of the GDN prefill kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

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
  // chunk table (written by the chunk-index builder)
  int32_t *chunk_idx;  // [cap][2]
  int32_t *cu_chunks;  // [N+1]
  int32_t *seq_bos;    // [N+1] sanitised sequence starts
  int32_t *n_chunks;   // [1]
  int32_t *chunk_tok;  // [cap][2] first token, length (0 for unused slots)
  int64_t cap;
  // intermediates
  void *Wf, *Kf, *Uf, *Hf, *Nf;
  float *Gw;
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
};

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

}  // namespace gdn
