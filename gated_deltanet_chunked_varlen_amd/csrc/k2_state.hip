// k2_state.hip -- inter-chunk state pass.
//
// Only the state crosses chunk boundaries (weigao.cc "GDN 与 Chunked
// Prefill", section "块内 state 和块间 final state"; 0539edu
// "GDN与线性注意力GPU并行实现", section 2.2: the chunk-level recurrence is
// serial over chunks and cheap for a few hundred of them).  Per chunk, with
// the chunk's W, U, Ktilde from the intra-chunk pass and S the state entering
// the chunk:
//
//   N  = U - W S                         (the chunk's new values)
//   S' = exp(G_last) S + Ktilde^T N
//
// Column v of S depends on column v of U (and of the initial state) only, so
// the state splits into independent 16-column tiles.  One wave64 owns one
// (sequence, sab head, 16-column tile): its 16 x D slice of S lives in
// registers in matrix-core result layout for the whole sequence, and the
// result registers of each product are the next product's operand (see the
// register-reuse note in gdn_common.h).  Per chunk it also stores the
// chunk-start state and N for the output pass, writes checkpoints (gitcode
// "FlashInfer GDN Prefill 完全指南", section "中间状态检查点") and, at the end,
// the final state into output_state (row state_indices[i] for a pool,
// section "状态池").
//
// Workgroup -> tile mapping: consecutive workgroup ids are dealt round-robin
// to the 8 XCDs, so the NT tiles of one (sequence, head) get ids equal mod 8
// and share one XCD's L2 for the W / Ktilde blocks they all read.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

__device__ __forceinline__ int64_t ld_index(const void *p, int type, int64_t i) {
  return type == GDN_I64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

template <typename T, int D>
__global__ void __launch_bounds__(64) state_kernel(Args a) {
  using M = Mfma<T>;
  using Ge = Geo<T, D>;
  typedef typename M::frag frag;
  constexpr int KPL = Ge::KPL, NT = Ge::NT, KS_D = Ge::KS_D, KS_C = Ge::KS_C;

  const int b = blockIdx.x;
  const int jv = (b >> 3) % NT;
  const int u = (b / (8 * NT)) * 8 + (b & 7);
  const int H = a.H;
  if (u >= a.N * H) return;
  const int seq = u / H, h = u % H;
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const int vcol = 16 * jv + c;

  const int f0 = a.cu_chunks[seq];
  const int nc = min(a.cu_chunks[seq + 1], a.n_chunks[0]) - f0;
  const int len = a.seq_bos[seq + 1] - a.seq_bos[seq];

  int64_t row = seq;
  bool row_ok = true;
  if (a.sidx) {
    row = ld_index(a.sidx, a.sidx_type, seq);
    row_ok = row >= 0 && row < a.pool_rows;
  }

  // S[it][r] = S[16 it + 4g + r][vcol]   (keys x values)
  float S[NT][4];
  if (a.init && row_ok) {
    const int64_t base = row * a.init_str[0] + (int64_t)h * a.init_str[1] + (int64_t)vcol * a.init_str[2];
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[it][r] = load_state_elem(a.init, a.init_dtype, base + (int64_t)(16 * it + 4 * g + r) * a.init_str[3]);
  } else {
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[it][r] = 0.f;
  }

  int64_t ck_base = 0;
  if (a.ck_every > 0) ck_base = ld_index(a.ck_cs, a.ck_cs_type, seq);

  for (int cc = 0; cc < nc; ++cc) {
    const int64_t ch = (int64_t)(f0 + cc) * H + h;
    // chunk-start state, dk in pi order
    {
      T *hf = (T *)a.Hf + ch * Ge::H_ELEMS + (int64_t)jv * KS_D * 64 * KPL;
#pragma unroll
      for (int kt = 0; kt < KS_D; ++kt) {
        frag v;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const int s = kt * KPL + e;
          M::set(v, e, S[s >> 2][s & 3]);
        }
        *reinterpret_cast<frag *>(hf + ((int64_t)kt * 64 + lane) * KPL) = v;
      }
    }
    // N = U - W S
    f32x4 acc[4];
    {
      const T *uf = (const T *)a.Uf + ch * Ge::W_ELEMS + (int64_t)jv * 4 * 64 * 4;
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[it][r] = to_f32(uf[((int64_t)it * 64 + lane) * 4 + r]);
      const T *wf = (const T *)a.Wf + ch * Ge::W_ELEMS;
#pragma unroll
      for (int kt = 0; kt < KS_D; ++kt) {
        frag bneg;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const int s = kt * KPL + e;
          M::set(bneg, e, -S[s >> 2][s & 3]);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const frag fa = *reinterpret_cast<const frag *>(wf + (((int64_t)it * KS_D + kt) * 64 + lane) * KPL);
          acc[it] = M::mma(fa, bneg, acc[it]);
        }
      }
    }
    // new values: operand fragments (t in pi order), stored for the output pass
    frag nf[KS_C];
    {
      T *nfp = (T *)a.Nf + ch * Ge::W_ELEMS + (int64_t)jv * KS_C * 64 * KPL;
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const int s = kt * KPL + e;
          M::set(nf[kt], e, acc[s >> 2][s & 3]);
        }
        *reinterpret_cast<frag *>(nfp + ((int64_t)kt * 64 + lane) * KPL) = nf[kt];
      }
    }
    // S' = exp(G_last) S + Ktilde^T N
    {
      const float gl = gexp(a.Gw[ch * kChunk + (kChunk - 1)]);
      const T *kf = (const T *)a.Kf + ch * Ge::W_ELEMS;
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        f32x4 s4 = {S[it][0] * gl, S[it][1] * gl, S[it][2] * gl, S[it][3] * gl};
#pragma unroll
        for (int kt = 0; kt < KS_C; ++kt) {
          const frag fa = *reinterpret_cast<const frag *>(kf + (((int64_t)it * KS_C + kt) * 64 + lane) * KPL);
          s4 = M::mma(fa, nf[kt], s4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) S[it][r] = s4[r];
      }
    }
    if (a.ck_every > 0) {
      const int done = (cc + 1) * kChunk;
      if (done <= len && done % a.ck_every == 0) {
        const int64_t crow = ck_base + done / a.ck_every - 1;
        if (crow >= 0 && crow < a.ck_rows) {
          const int64_t base = crow * a.ck_str[0] + (int64_t)h * a.ck_str[1] + (int64_t)vcol * a.ck_str[2];
#pragma unroll
          for (int it = 0; it < NT; ++it)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              store_state_elem(a.ck, a.ck_dtype, base + (int64_t)(16 * it + 4 * g + r) * a.ck_str[3], S[it][r]);
        }
      }
    }
  }

  if (a.out_final && a.outst && row_ok) {
    const int64_t base = row * a.out_str[0] + (int64_t)h * a.out_str[1] + (int64_t)vcol * a.out_str[2];
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store_state_elem(a.outst, a.out_dtype, base + (int64_t)(16 * it + 4 * g + r) * a.out_str[3], S[it][r]);
  }
}

template <typename T, int D>
static hipError_t launch_state_t(const Args &a, hipStream_t s) {
  constexpr int NT = D / 16;
  const int64_t units = (int64_t)a.N * a.H;
  if (units == 0) return hipSuccess;
  const int64_t blocks = ((units + 7) / 8) * 8 * NT;
  state_kernel<T, D><<<dim3((unsigned)blocks), dim3(64), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_state(const Args &a, hipStream_t s) {
  if (a.dtype == GDN_BF16) {
    if (a.D == 128) return launch_state_t<bf16, 128>(a, s);
    if (a.D == 64) return launch_state_t<bf16, 64>(a, s);
    return launch_state_t<bf16, 32>(a, s);
  }
  if (a.D == 128) return launch_state_t<float, 128>(a, s);
  if (a.D == 64) return launch_state_t<float, 64>(a, s);
  return launch_state_t<float, 32>(a, s);
}

}  // namespace gdn
