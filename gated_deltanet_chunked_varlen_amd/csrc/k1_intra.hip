// k1_intra.hip -- intra-chunk pass: everything about one 64-token chunk of
// one head that does not depend on the state entering the chunk.
//
// weigao.cc "GDN 与 Chunked Prefill", section "为什么要切成 64-token chunk"
// (the chunk's work is a cumsum, a triangular solve and a recompute) and
// section "递推公式如何展开成块内计算" (the decay table of the unrolled
// recurrence).  With G_t the cumulative sum of log alpha inside the chunk:
//
//   A[t][j] = beta_t exp(G_t - G_j) (k_t . k_j)   for j < t, else 0
//   T       = (I + A)^{-1}                          (unit lower triangular)
//   W       = T diag(beta exp(G)) K,   U = T diag(beta) V
//   Ktilde  = diag(exp(G_last - G)) K
//
// so that the state pass can do N = U - W S and S' = exp(G_last) S +
// Ktilde^T N per chunk.
//
// One workgroup of four wave64s per (flat chunk, sab head).  Rows of the
// chunk beyond the sequence end act as alpha = 1, beta = 0, k = v = 0, which
// leaves every product exact.  T is computed in fp32: the 16x16 diagonal
// blocks by forward substitution, the off-diagonal blocks row block by row
// block on the fp32 matrix cores (T_ij = -T_ii sum_m A_im T_mj).  W, U and
// Ktilde^T leave in the fragment-major layouts of gdn_common.h.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

template <typename T> struct Pad { static constexpr int v = 16 / sizeof(T); };

template <typename T, int D>
struct IntraSmem {
  T Ks[64][D + Pad<T>::v];        // k rows (normalised), natural order
  T KsT[D][64 + Pad<T>::v];       // the same, transposed
  T VsT[D][64 + Pad<T>::v];       // v, transposed
  float Am[64][64 + 4];
  float Tm[64][64 + 4];
  float Gs[64];
  float Bs[64];
};

template <typename T, int D>
__global__ void __launch_bounds__(256) intra_kernel(Args a) {
  using M = Mfma<T>;
  using Ge = Geo<T, D>;
  constexpr int KPL = Ge::KPL, NT = Ge::NT, KS_D = Ge::KS_D, KS_C = Ge::KS_C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IntraSmem<T, D> &sm = *reinterpret_cast<IntraSmem<T, D> *>(smem_raw);

  const int64_t ch = blockIdx.x;
  const int H = a.H;
  const int f = (int)(ch / H), h = (int)(ch % H);
  if (f >= a.n_chunks[0]) return;
  const int seq = a.chunk_idx[2 * f], cidx = a.chunk_idx[2 * f + 1];
  const int64_t bos = (int64_t)a.seq_bos[seq] + (int64_t)kChunk * cidx;
  const int len = (int)min<int64_t>(kChunk, (int64_t)a.seq_bos[seq + 1] - bos);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;

  // ---- load k (normalised), v; gates ------------------------------------
  {
    const int t = tid >> 2, p = tid & 3;
    const bool valid = t < len;
    const int kh = h / (H / a.hk), vh = h / (H / a.hv);
    float x[D / 4];
    if (valid) {
      const T *row = (const T *)a.k + ((bos + t) * a.hk + kh) * D;
      load_row_part<T, D>(row, p, x);
    } else {
#pragma unroll
      for (int e = 0; e < D / 4; ++e) x[e] = 0.f;
    }
    float inv = 1.f;
    if (a.l2norm) inv = row_inv_norm<D>(x);
#pragma unroll
    for (int e = 0; e < D / 4; ++e) {
      const int col = row_part_idx(p, e);
      const T val = from_f32<T>(x[e] * inv);
      sm.Ks[t][col] = val;
      sm.KsT[col][t] = val;
    }
    if (valid) {
      const T *row = (const T *)a.v + ((bos + t) * a.hv + vh) * D;
      load_row_part<T, D>(row, p, x);
    } else {
#pragma unroll
      for (int e = 0; e < D / 4; ++e) x[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < D / 4; ++e) sm.VsT[row_part_idx(p, e)][t] = from_f32<T>(x[e]);
  }
  if (wave == 0) {
    const int t = lane;
    const bool valid = t < len;
    float la = 0.f, be = 0.f;
    if (valid) {
      const int64_t gi = (bos + t) * H + h;
      la = a.g ? logf(a.g[gi]) : 0.f;
      be = a.beta ? a.beta[gi] : 1.f;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(la, o);
      if (lane >= o) la += y;
    }
    sm.Gs[t] = la;
    sm.Bs[t] = be;
    a.Gw[ch * kChunk + t] = la;
  }
  __syncthreads();

  // ---- A = strictly-lower(beta_t exp(G_t - G_j) k_t.k_j) ------------------
  {
    const int it = wave;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (jt <= it) {
#pragma unroll
        for (int kt = 0; kt < KS_D; ++kt) {
          const int k0 = kt * 4 * KPL + g * KPL;
          const typename M::frag fa = *reinterpret_cast<const typename M::frag *>(&sm.Ks[16 * it + c][k0]);
          const typename M::frag fb = *reinterpret_cast<const typename M::frag *>(&sm.Ks[16 * jt + c][k0]);
          acc = M::mma(fa, fb, acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * it + 4 * g + r, j = 16 * jt + c;
        sm.Am[t][j] = (j < t) ? sm.Bs[t] * gexp(sm.Gs[t] - sm.Gs[j]) * acc[r] : 0.f;
      }
    }
  }
  __syncthreads();

  // ---- T = (I + A)^{-1}: diagonal blocks --------------------------------
  {
    const int bw = wave;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(-sm.Am[16 * bw + i][16 * bw + m], tc[m], s);
      tc[i] = (i < c) ? 0.f : s;
    }
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.Tm[16 * bw + i][16 * bw + c] = tc[i];
    }
    // zero the blocks above the diagonal
    for (int e = lane; e < 16 * 64; e += 64) {
      const int i = e >> 6, j = e & 63;
      if (j >= 16 * (bw + 1)) sm.Tm[16 * bw + i][j] = 0.f;
    }
  }
  __syncthreads();
  // ---- off-diagonal blocks, one row block at a time ----------------------
#pragma unroll
  for (int bi = 1; bi < 4; ++bi) {
    const int bj = wave;
    if (bj < bi) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int m = bj; m < bi; ++m) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const float fa = sm.Am[16 * bi + c][16 * m + 4 * kt + g];
          const float fb = sm.Tm[16 * m + 4 * kt + g][16 * bj + c];
          x = Mfma<float>::mma(fa, fb, x);
        }
      }
      // T_ij = -T_ii X; X rows 4g..4g+3 sit in this lane group: contract over
      // them in pi order (slot kt of group g is row 4g + kt).
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float fa = sm.Tm[16 * bi + c][16 * bi + 4 * g + kt];
        y = Mfma<float>::mma(fa, x[kt], y);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.Tm[16 * bi + 4 * g + r][16 * bj + c] = -y[r];
    }
    __syncthreads();
  }

  // ---- W (as W^T tiles) -------------------------------------------------
  const int w = wave;  // token tile of this wave
  {
    typename M::frag bw[KS_C];
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int j = kt * 4 * KPL + g * KPL + e;
        M::set(bw[kt], e, sm.Tm[16 * w + c][j] * sm.Bs[j] * gexp(sm.Gs[j]));
      }
    }
    T *wf = (T *)a.Wf + ch * Ge::W_ELEMS + (int64_t)w * KS_D * 64 * KPL;
    typename M::frag out[KS_D];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
        const typename M::frag fa =
            *reinterpret_cast<const typename M::frag *>(&sm.KsT[16 * dt + c][kt * 4 * KPL + g * KPL]);
        acc = M::mma(fa, bw[kt], acc);
      }
      // lane holds W[16w + c][16dt + 4g + r] = slot s = 4dt + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 4 * dt + r;
        M::set(out[s / KPL], s % KPL, acc[r]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt)
      *reinterpret_cast<typename M::frag *>(wf + ((int64_t)kt * 64 + lane) * KPL) = out[kt];
  }
  // ---- U ------------------------------------------------------------------
  {
    typename M::frag au[KS_C];
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int j = kt * 4 * KPL + g * KPL + e;
        M::set(au[kt], e, sm.Tm[16 * w + c][j] * sm.Bs[j]);
      }
    }
    T *uf = (T *)a.Uf + ch * Ge::W_ELEMS;
#pragma unroll
    for (int jv = 0; jv < NT; ++jv) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
        const typename M::frag fb =
            *reinterpret_cast<const typename M::frag *>(&sm.VsT[16 * jv + c][kt * 4 * KPL + g * KPL]);
        acc = M::mma(au[kt], fb, acc);
      }
      T *dst = uf + (((int64_t)jv * 4 + w) * 64 + lane) * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = from_f32<T>(acc[r]);
    }
  }
  // ---- Ktilde^T fragments ---------------------------------------------------
  {
    const float glast = sm.Gs[63];
    T *kf = (T *)a.Kf + ch * Ge::W_ELEMS;
    constexpr int NFRAG = NT * KS_C * 64;
    for (int fi = tid; fi < NFRAG; fi += 256) {
      const int fl = fi & 63, kt = (fi >> 6) % KS_C, it2 = (fi >> 6) / KS_C;
      const int fg = fl >> 4, fc = fl & 15;
      typename M::frag v;
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int j = pi_idx(fg, kt * KPL + e);
        M::set(v, e, to_f32(sm.KsT[16 * it2 + fc][j]) * gexp(glast - sm.Gs[j]));
      }
      *reinterpret_cast<typename M::frag *>(kf + (int64_t)fi * KPL) = v;
    }
  }
}

template <typename T, int D>
static hipError_t launch_intra_t(const Args &a, hipStream_t s) {
  const size_t smem = sizeof(IntraSmem<T, D>);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)intra_kernel<T, D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = a.cap * a.H;
  if (blocks == 0) return hipSuccess;
  intra_kernel<T, D><<<dim3((unsigned)blocks), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_intra(const Args &a, hipStream_t s) {
  if (a.dtype == GDN_BF16) {
    if (a.D == 128) return launch_intra_t<bf16, 128>(a, s);
    if (a.D == 64) return launch_intra_t<bf16, 64>(a, s);
    return launch_intra_t<bf16, 32>(a, s);
  }
  if (a.D == 128) return launch_intra_t<float, 128>(a, s);
  if (a.D == 64) return launch_intra_t<float, 64>(a, s);
  return launch_intra_t<float, 32>(a, s);
}

}  // namespace gdn
