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
//   W       = T diag(beta exp(G)) K,   U = T diag(beta) V   (W stored as -W)
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

// LDS plan of the fp32 variant (intra_kernel; 16-bit inputs take
// intra_kernel_h below): about 85 KB at D = 128, one workgroup per CU.  k rows
// are needed only for K K^T, v (transposed) only after it, so they share
// storage; A is inverted in place into T; the two spare columns of the padded
// A/T rows hold G and beta.
template <typename T, int D>
struct IntraSmem {
  union {
    T Ks[64][D + Pad<T>::v];      // k rows (normalised), natural order
    T VsT[D][64 + Pad<T>::v];     // v, transposed
  } kv;
  T KsT[D][64 + Pad<T>::v];       // k (normalised), transposed
  float AT[64][64 + 4];           // A, then T in place; [t][64] = G, [t][65] = beta
};

template <typename T, int D>
__global__ void __launch_bounds__(256) intra_kernel(Args a) {
  using M = Mfma<T>;
  using Ge = Geo<T, D>;
  constexpr int KPL = Ge::KPL, NT = Ge::NT, KS_D = Ge::KS_D, KS_C = Ge::KS_C;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IntraSmem<T, D> &sm = *reinterpret_cast<IntraSmem<T, D> *>(smem_raw);

  const int H = a.H;
  const int f = (int)(blockIdx.x / H), h = (int)(blockIdx.x % H);
  const int64_t ch = ws_index(f, h, a.cap);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tb, len;
  chunk_geometry(a, f, lane, blockIdx.x == 0 && wave == 0, tb, len);
  if (len <= 0) return;
  const int64_t bos = tb;

  const int g = lane >> 4, c = lane & 15;
  float(*AT)[68] = sm.AT;

  // ---- load k (normalised) and v; gates ----------------------------------
  const int lt = tid >> 2, lp = tid & 3;   // row and row part of this thread
  float vx[D / 4];
  {
    const bool valid = lt < len;
    const int kh = h / (H / a.hk), vh = h / (H / a.hv);
    float x[D / 4];
    if (valid) {
      load_row_part<T, D>((const T *)a.k + ((bos + lt) * a.hk + kh) * D, lp, x);
      load_row_part<T, D>((const T *)a.v + ((bos + lt) * a.hv + vh) * D, lp, vx);
    } else {
#pragma unroll
      for (int e = 0; e < D / 4; ++e) x[e] = vx[e] = 0.f;
    }
    float inv = 1.f;
    if (a.l2norm) inv = row_inv_norm<D>(x);
#pragma unroll
    for (int e = 0; e < D / 4; ++e) {
      const int col = row_part_idx(lp, e);
      const T val = from_f32<T>(x[e] * inv);
      sm.kv.Ks[lt][col] = val;
      sm.KsT[col][lt] = val;
    }
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
    la = wave_prefix_sum(la);
    AT[t][64] = la;
    AT[t][65] = be;
    a.Gw[ch * kChunk + t] = la;
  }
  lds_sync();

  // ---- A = strictly-lower(beta_t exp(G_t - G_j) k_t.k_j) ------------------
  {
    const int it = wave;
    f32x4 acc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jt <= it) {
#pragma unroll
        for (int kt = 0; kt < KS_D; ++kt) {
          const int k0 = kt * 4 * KPL + g * KPL;
          const typename M::frag fa = *reinterpret_cast<const typename M::frag *>(&sm.kv.Ks[16 * it + c][k0]);
          const typename M::frag fb = *reinterpret_cast<const typename M::frag *>(&sm.kv.Ks[16 * jt + c][k0]);
          acc[jt] = M::mma(fa, fb, acc[jt]);
        }
      }
    }
    float Gt[4], Bt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Gt[r] = AT[16 * it + 4 * g + r][64];
      Bt[r] = AT[16 * it + 4 * g + r][65];
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = 16 * jt + c;
      const float Gj = AT[j][64];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * it + 4 * g + r;
        AT[t][j] = (j < t) ? Bt[r] * gexp(Gt[r] - Gj) * acc[jt][r] : 0.f;
      }
    }
  }
  lds_sync();

  // ---- v into LDS (transposed, over the k rows); T diagonal blocks -------
#pragma unroll
  for (int e = 0; e < D / 4; ++e) sm.kv.VsT[row_part_idx(lp, e)][lt] = from_f32<T>(vx[e]);
  {
    const int bw = wave;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(-AT[16 * bw + i][16 * bw + m], tc[m], s);
      tc[i] = (i < c) ? 0.f : s;
    }
    // every lane has read its A block: overwrite it with T (upper part 0)
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) AT[16 * bw + i][16 * bw + c] = tc[i];
    }
  }
  lds_sync();
  // ---- off-diagonal blocks, one row block at a time ----------------------
#pragma unroll
  for (int bi = 1; bi < 4; ++bi) {
    const int bj = wave;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (bj < bi) {
      // X = sum_m A_{bi,m} T_{m,bj}; row block bi still holds A
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int m = bj; m < bi; ++m) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          x = Mfma<float>::mma(AT[16 * bi + c][16 * m + 4 * kt + g],
                               AT[16 * m + 4 * kt + g][16 * bj + c], x);
      }
      // T_ij = -T_ii X; X rows 4g..4g+3 sit in this lane group: contract over
      // them in pi order (slot kt of group g is row 4g + kt).
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        y = Mfma<float>::mma(AT[16 * bi + c][16 * bi + 4 * g + kt], x[kt], y);
    }
    lds_sync();  // all reads of row block bi's A are done
    if (bj < bi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) AT[16 * bi + 4 * g + r][16 * bj + c] = -y[r];
    }
    lds_sync();
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
        M::set(bw[kt], e, AT[16 * w + c][j] * AT[j][65] * gexp(AT[j][64]));
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
      // lane holds W[16w + c][16dt + 4g + r] = slot s = 4dt + r; stored
      // negated so the state pass accumulates U + (-W) S directly
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 4 * dt + r;
        M::set(out[s / KPL], s % KPL, -acc[r]);
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
        M::set(au[kt], e, AT[16 * w + c][j] * AT[j][65]);
      }
    }
    T *uf = (T *)a.Uf + ch * Ge::W_ELEMS;
#pragma unroll
    for (int jv = 0; jv < NT; ++jv) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
        const typename M::frag fb =
            *reinterpret_cast<const typename M::frag *>(&sm.kv.VsT[16 * jv + c][kt * 4 * KPL + g * KPL]);
        acc = M::mma(au[kt], fb, acc);
      }
      T *dst = uf + (((int64_t)jv * 4 + w) * 64 + lane) * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[r] = from_f32<T>(acc[r]);
    }
  }
  // ---- Ktilde^T fragments ---------------------------------------------------
  {
    const float glast = AT[63][64];
    T *kf = (T *)a.Kf + ch * Ge::W_ELEMS;
    constexpr int NFRAG = NT * KS_C * 64;
    for (int fi = tid; fi < NFRAG; fi += 256) {
      const int fl = fi & 63, kt = (fi >> 6) % KS_C, it2 = (fi >> 6) / KS_C;
      const int fg = fl >> 4, fc = fl & 15;
      typename M::frag v;
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int j = pi_idx(fg, kt * KPL + e);
        M::set(v, e, to_f32(sm.KsT[16 * it2 + fc][j]) * gexp(glast - AT[j][64]));
      }
      *reinterpret_cast<typename M::frag *>(kf + (int64_t)fi * KPL) = v;
    }
  }
}

template <typename T, int D>
static hipError_t launch_intra_t(const Args &a, hipStream_t s) {
  const size_t smem = sizeof(IntraSmem<T, D>);
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = set_dynamic_lds((const void *)intra_kernel<T, D>, (int)smem, lds_set);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = a.cap * a.H;
  if (blocks == 0) return hipSuccess;
  intra_kernel<T, D><<<dim3((unsigned)blocks), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// 16-bit (bf16 / fp16) variant.  k and v stay row-major in LDS and every product that
// contracts over the chunk's rows reads them through transposed LDS reads
// (lds_col_frag), so there is no transposed copy: one padded 64 x D bf16
// buffer holds the normalised k rows and, once W and Ktilde^T are out, the v
// rows.  With the fp32 A/T buffer that is about 35 KB at D = 128, and four
// workgroups share a CU.  The chunk's first token and length come from the
// (first token, length) table in one load.
// ---------------------------------------------------------------------------
// A store of an intermediate: non-temporal when the intermediates outgrow the
// last-level cache (NT), plain otherwise.  NT is a template parameter: with a
// run-time flag the compiler merges the two stores and drops the hint.
template <bool NT, typename V>
__device__ __forceinline__ void st_inter(V *p, const V &v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <typename T, int D>
struct IntraSmemB {
  static constexpr int LDK = D + 16;  // row pitch in elements (32 B pad)
  T KV[64][LDK];                   // normalised k rows, later v rows
  float AT[64][68];                   // A, then T; [t][64] = G, [t][65] = beta
};

template <typename T, int D, bool NTS, bool SHK, bool TF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) intra_kernel_h(Args a) {
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int NT = D / 16, KS_D = D / 32, KS_C = 2, NV = D / 32;
  constexpr int LDK = IntraSmemB<T, D>::LDK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IntraSmemB<T, D> &sm = *reinterpret_cast<IntraSmemB<T, D> *>(smem_raw);

  const int H = a.H;
  const int f = (int)(blockIdx.x / H), h = (int)(blockIdx.x % H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tb, len;
  chunk_geometry(a, f, lane, blockIdx.x == 0 && wave == 0, tb, len);
  if (len <= 0) return;
  const int64_t bos = tb;
  const int64_t ch = ws_index(f, h, a.cap);

  const int g = lane >> 4, c = lane & 15;
  float(*AT)[68] = sm.AT;
  T(*KV)[LDK] = sm.KV;

  // ---- k (normalised) into LDS, v kept in registers; gates ---------------
  const int lt = tid >> 2, lp = tid & 3;  // row and row part of this thread
  u32x4 vraw[NV];
  {
    const bool valid = lt < len;
    const int kh = h / (H / a.hk), vh = h / (H / a.hv);
    const T *vrow = (const T *)a.v + ((bos + lt) * a.hv + vh) * D;
#pragma unroll
    for (int i = 0; i < NV; ++i)
      vraw[i] = (valid && !TF) ? *reinterpret_cast<const u32x4 *>(vrow + 32 * i + 8 * lp)
                               : u32x4{0, 0, 0, 0};
    frag kn[NV];
    float kinv;
    load_norm_row16<T, D>((const T *)a.k + ((bos + lt) * a.hk + kh) * D, lp, valid,
                          a.l2norm != 0, kn, &kinv);
#pragma unroll
    for (int i = 0; i < NV; ++i) *reinterpret_cast<frag *>(&KV[lt][32 * i + 8 * lp]) = kn[i];
    // T form: the k row's normalisation factor (0 past the chunk's end) in
    // column 66 of the A/T buffer, beside the gate and beta columns
    if (TF && lp == 0) AT[lt][66] = valid ? kinv : 0.f;
    if (a.fuse) {
      // q rows (normalised) go to the A/T buffer until A is formed: row t at
      // byte 272 t, below the G / beta columns (bytes 256 .. 263 of the row)
      const int qh = h / (H / a.hq);
      frag qn[NV];
      load_norm_row16<T, D>((const T *)a.q + ((bos + lt) * a.hq + qh) * D, lp, valid,
                            a.l2norm != 0, qn);
      T *qrow = reinterpret_cast<T *>(&AT[lt][0]);
#pragma unroll
      for (int i = 0; i < NV; ++i) *reinterpret_cast<frag *>(qrow + 32 * i + 8 * lp) = qn[i];
    }
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
    la = wave_prefix_sum(la);
    AT[t][64] = la;
    AT[t][65] = be;
    a.Gw[ch * kChunk + t] = la;
  }
  lds_sync();

  if (a.fuse) {
    // ---- operands of the output products, for the fused state pass --------
    // Pf [tt][kt]: P[16 tt + c][pi(g, 8 kt + e)] with P = (Q K^T) masked to
    //   j <= t and scaled by exp(G_t - G_j) (P^T = K Q^T leaves P rows in the
    //   operand order); Qf [tt][kt]: q[16 tt + c][pi(g, 8 kt + e)].
    const int tt = wave;
    const T(*QR)[136] = reinterpret_cast<const T(*)[136]>(&AT[0][0]);
    T *pf_out = (T *)a.Pf + ch * (int64_t)(64 * 64);
    // q fragments once per q head (the first sab head that reads it writes)
    T *qf_out = (T *)a.Qf + q_block(a, ch, h) * (int64_t)(64 * D);
    const bool write_q = h % (H / a.hq) == 0;
    frag pf[KS_C];
    const int t = 16 * tt + c;
    const float gt = AT[t][64];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (jt <= tt) {
#pragma unroll
        for (int kt = 0; kt < KS_D; ++kt) {
          const int k0 = kt * 32 + g * 8;
          const frag fa = *reinterpret_cast<const frag *>(&KV[16 * jt + c][k0]);
          const frag fb = *reinterpret_cast<const frag *>(&QR[16 * tt + c][k0]);
          acc = M::mma(fa, fb, acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * g + r;
        const float pv = (j <= t) ? acc[r] * gexp(gt - AT[j][64]) : 0.f;
        const int sl = 4 * jt + r;
        pf[sl / 8][sl % 8] = (T)pv;
      }
    }
    // the blocks with 2 kt > tt are all zero; the fused pass does not read them
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt)
      if (2 * kt <= tt)
        st_inter<NTS>(reinterpret_cast<frag *>(pf_out + (((int64_t)tt * KS_C + kt) * 64 + lane) * 8), pf[kt]);
    if (write_q) {
#pragma unroll
      for (int kt = 0; kt < KS_D; ++kt) {
        frag qf;
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] = QR[t][pi_idx(g, kt * 8 + e)];
        st_inter<NTS>(reinterpret_cast<frag *>(qf_out + (((int64_t)tt * KS_D + kt) * 64 + lane) * 8), qf);
      }
    }
    lds_sync();  // q is consumed: A may overwrite the buffer
  }

  // ---- A = strictly-lower(beta_t exp(G_t - G_j) k_t.k_j) ------------------
  {
    const int it = wave;
    f32x4 acc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jt <= it) {
#pragma unroll
        for (int kt = 0; kt < KS_D; ++kt) {
          const int k0 = kt * 32 + g * 8;
          const frag fa = *reinterpret_cast<const frag *>(&KV[16 * it + c][k0]);
          const frag fb = *reinterpret_cast<const frag *>(&KV[16 * jt + c][k0]);
          acc[jt] = M::mma(fa, fb, acc[jt]);
        }
      }
    }
    float Gt[4], Bt[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      Gt[r] = AT[16 * it + 4 * g + r][64];
      Bt[r] = AT[16 * it + 4 * g + r][65];
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = 16 * jt + c;
      const float Gj = AT[j][64];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * it + 4 * g + r;
        AT[t][j] = (j < t) ? Bt[r] * gexp(Gt[r] - Gj) * acc[jt][r] : 0.f;
      }
    }
  }
  lds_sync();

  // ---- T diagonal blocks (forward substitution, lane c = column c) --------
  {
    const int bw = wave;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float s = (i == c) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) s = fmaf(-AT[16 * bw + i][16 * bw + m], tc[m], s);
      tc[i] = (i < c) ? 0.f : s;
    }
    if (g == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) AT[16 * bw + i][16 * bw + c] = tc[i];
    }
  }
  lds_sync();
  // ---- off-diagonal blocks, one row block at a time ----------------------
#pragma unroll
  for (int bi = 1; bi < 4; ++bi) {
    const int bj = wave;
    f32x4 y = {0.f, 0.f, 0.f, 0.f};
    if (bj < bi) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      for (int m = bj; m < bi; ++m) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          x = Mfma<float>::mma(AT[16 * bi + c][16 * m + 4 * kt + g],
                               AT[16 * m + 4 * kt + g][16 * bj + c], x);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        y = Mfma<float>::mma(AT[16 * bi + c][16 * bi + 4 * g + kt], x[kt], y);
    }
    lds_sync();
    if (bj < bi) {
#pragma unroll
      for (int r = 0; r < 4; ++r) AT[16 * bi + 4 * g + r][16 * bj + c] = -y[r];
    }
    lds_sync();
  }

  const int w = wave;  // token tile of this wave
  if constexpr (TF) {
    // ---- T form: -T diag(beta) and the row scales ----------------------------
    // The state pass forms N = U - W S = T diag(beta) (V - diag(exp(G) / |k|)
    // (K S)) from the raw k and v rows, so instead of -W and U this stores
    // the 64 x 64 factor -T diag(beta) as operand fragments: [w][kt][lane] =
    // rows 16 w + c, columns (tokens) in pi order, matching the pi order of
    // the products' result rows; and per token exp(G_t) / |k_t| and
    // exp(G_last - G_t) / |k_t| (Ktilde^T N = K^T diag(that) N).  v is not
    // read here at all.
    T *tf = (T *)a.Wf + ch * (int64_t)(64 * 64) + (int64_t)w * KS_C * 64 * 8;
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
      // rows 0 .. 31 have no columns 32 .. 63 (T is lower triangular): those
      // two fragments are neither stored here nor read by the state pass
      if (kt > 0 && w < 2) continue;
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * kt + 16 * (e >> 2) + 4 * g + (e & 3);
        y[e] = -AT[16 * w + c][j] * AT[j][65];
      }
      st_inter<NTS>(reinterpret_cast<frag *>(tf + ((int64_t)kt * 64 + lane) * 8), M::pack(y));
    }
    if (wave == 0) {
      const float inv = AT[lane][66], gt = AT[lane][64];
      float *bw = a.Bw + ch * 128;
      bw[lane] = gexp(gt) * inv;
      bw[64 + lane] = gexp(AT[63][64] - gt) * inv;
    }
    return;
  } else {
  // ---- W (as W^T tiles): A operand = k columns via transposed reads --------
  {
    frag bw[KS_C];
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = kt * 32 + g * 8 + e;
        y[e] = AT[16 * w + c][j] * AT[j][65] * gexp(AT[j][64]);
      }
      bw[kt] = M::pack(y);
    }
    T *wf = (T *)a.Wf + ch * (int64_t)(64 * D) + (int64_t)w * KS_D * 64 * 8;
    frag out[KS_D];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
        const frag fa = lds_col_frag(&KV[0][0], LDK, kt * 32 + g * 8, kt * 32 + g * 8 + 4, 16 * dt, c);
        acc = M::mma(fa, bw[kt], acc);
      }
      // lane holds W[16w + c][16dt + 4g + r] = slot s = 4dt + r; stored
      // negated so the state pass accumulates U + (-W) S directly
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 4 * dt + r;
        out[s / 8][s % 8] = (T)(-acc[r]);
      }
    }
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt)
      st_inter<NTS>(reinterpret_cast<frag *>(wf + ((int64_t)kt * 64 + lane) * 8), out[kt]);
  }
  // ---- K^T fragments: rows pi(g, 8kt + e) of k column 16 it2 + c ----------
  // Where sab heads share a k head, the normalised k once per k head (the
  // first sab head that reads it writes), and the state pass applies each sab
  // head's decay to the chunk end, exp(G_last - G_t), to N's rows instead
  // (Ktilde^T N = K^T diag(.) N); otherwise Ktilde^T itself.
  if (h % (H / a.hk) == 0) {
    constexpr bool shared = SHK;  // sab heads share k heads
    const float glast = AT[63][64];
    T *kf = (T *)a.Kf + k_block(a, ch, h) * (int64_t)(64 * D);
#pragma unroll
    for (int q = 0; q < NT * KS_C / 4; ++q) {
      const int fidx = wave + 4 * q;  // fragment block (row tile it2, k-step kt)
      const int kt = fidx % KS_C, it2 = fidx / KS_C;
      const int r0 = 32 * kt + 4 * g, r1 = r0 + 16;
      frag kv = lds_col_frag(&KV[0][0], LDK, r0, r1, 16 * it2, c);
      if (!shared) {
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = (e < 4 ? r0 : r1) + (e & 3);
          y[e] = (float)kv[e] * gexp(glast - AT[j][64]);
        }
        kv = M::pack(y);
      }
      st_inter<NTS>(reinterpret_cast<frag *>(kf + ((int64_t)fidx * 64 + lane) * 8), kv);
    }
  }
  }  // W form
  lds_sync();  // k rows consumed
#pragma unroll
  for (int i = 0; i < NV; ++i) *reinterpret_cast<u32x4 *>(&KV[lt][32 * i + 8 * lp]) = vraw[i];
  lds_sync();
  // ---- U ------------------------------------------------------------------
  {
    frag au[KS_C];
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = kt * 32 + g * 8 + e;
        y[e] = AT[16 * w + c][j] * AT[j][65];
      }
      au[kt] = M::pack(y);
    }
    T *uf = (T *)a.Uf + ch * (int64_t)(64 * D);
#pragma unroll
    for (int jv = 0; jv < NT; ++jv) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
        const frag fb = lds_col_frag(&KV[0][0], LDK, kt * 32 + g * 8, kt * 32 + g * 8 + 4, 16 * jv, c);
        acc = M::mma(au[kt], fb, acc);
      }
      T *dst = uf + (((int64_t)jv * 4 + w) * 64 + lane) * 4;
      typename M::half o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = (T)acc[r];
      st_inter<NTS>(reinterpret_cast<typename M::half *>(dst), o4);
    }
  }
}

// ---------------------------------------------------------------------------
// T form where R = H / hk = H / hq sab heads (2 .. 4) share each q and k head
// (GVA: two v heads per q/k head).  One workgroup per (chunk, q/k head) loads
// and normalises the q and k rows once and forms the raw Q K^T and K K^T
// products once; then, for each of its R sab heads in turn, it applies that
// head's gates and beta (P, A), inverts I + A and stores -T diag(beta) and
// the row scales, as the one-head T form does.  The q and k loads were half
// of a one-head workgroup's life.
// ---------------------------------------------------------------------------
template <typename T, int D>
struct IntraSmemS {
  IntraSmemB<T, D> b;
  float G[4][64], B[4][64], inv[64];  // per sab head gate log-cumsum, beta; 1/|k|
};

template <typename T, int D, bool NTS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
intra_tform_shared_kernel(Args a) {
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int KS_D = D / 32, KS_C = 2, NV = D / 32;
  constexpr int LDK = IntraSmemB<T, D>::LDK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  IntraSmemS<T, D> &sm = *reinterpret_cast<IntraSmemS<T, D> *>(smem_raw);
  float(*AT)[68] = sm.b.AT;
  T(*KV)[LDK] = sm.b.KV;

  const int H = a.H, R = H / a.hk;
  const int f = (int)(blockIdx.x / a.hk), kh = (int)(blockIdx.x % a.hk);
  const int h0 = kh * R;  // first sab head of this q/k head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tb, len;
  chunk_geometry(a, f, lane, blockIdx.x == 0 && wave == 0, tb, len);
  if (len <= 0) return;
  const int64_t bos = tb;
  const int g = lane >> 4, c = lane & 15;

  // ---- normalised k rows and q rows into LDS; per-head gates ---------------
  const int lt = tid >> 2, lp = tid & 3;
  {
    const bool valid = lt < len;
    frag kn[NV], qn[NV];
    float kinv;
    load_norm_row16<T, D>((const T *)a.k + ((bos + lt) * a.hk + kh) * D, lp, valid,
                          a.l2norm != 0, kn, &kinv);
    load_norm_row16<T, D>((const T *)a.q + ((bos + lt) * a.hq + kh) * D, lp, valid,
                          a.l2norm != 0, qn);
    // q rows in the A/T buffer until the first head's A is formed
    T *qrow = reinterpret_cast<T *>(&AT[lt][0]);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      *reinterpret_cast<frag *>(&KV[lt][32 * i + 8 * lp]) = kn[i];
      *reinterpret_cast<frag *>(qrow + 32 * i + 8 * lp) = qn[i];
    }
    if (lp == 0) sm.inv[lt] = valid ? kinv : 0.f;
  }
  if (wave < R) {
    // wave r: gate log-cumsum and beta of sab head h0 + r
    const int h = h0 + wave, t = lane;
    const bool valid = t < len;
    float la = 0.f, be = 0.f;
    if (valid) {
      const int64_t gi = (bos + t) * H + h;
      la = a.g ? logf(a.g[gi]) : 0.f;
      be = a.beta ? a.beta[gi] : 1.f;
    }
    la = wave_prefix_sum(la);
    sm.G[wave][t] = la;
    sm.B[wave][t] = be;
    a.Gw[ws_index(f, h, a.cap) * kChunk + t] = la;
  }
  lds_sync();

  // ---- raw Q K^T (token tile tt = wave) and K K^T (row tile it = wave) -----
  const int tt = wave, it = wave;
  f32x4 qk[4], kk[4];
  {
    const T(*QR)[136] = reinterpret_cast<const T(*)[136]>(&AT[0][0]);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      qk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      kk[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (jt <= tt) {
#pragma unroll
        for (int kt = 0; kt < KS_D; ++kt) {
          const int k0 = kt * 32 + g * 8;
          const frag fk = *reinterpret_cast<const frag *>(&KV[16 * jt + c][k0]);
          qk[jt] = M::mma(fk, *reinterpret_cast<const frag *>(&QR[16 * tt + c][k0]), qk[jt]);
          kk[jt] = M::mma(*reinterpret_cast<const frag *>(&KV[16 * it + c][k0]), fk, kk[jt]);
        }
      }
    }
    // q fragments, once for the q head
    T *qf_out = (T *)a.Qf + q_block(a, ws_index(f, h0, a.cap), h0) * (int64_t)(64 * D);
    const int t = 16 * tt + c;
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt) {
      frag qf;
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[e] = QR[t][pi_idx(g, kt * 8 + e)];
      st_inter<NTS>(reinterpret_cast<frag *>(qf_out + (((int64_t)tt * KS_D + kt) * 64 + lane) * 8), qf);
    }
  }

  for (int r = 0; r < R; ++r) {
    const int h = h0 + r;
    const int64_t ch = ws_index(f, h, a.cap);
    const float *Gr = sm.G[r], *Br = sm.B[r];
    // ---- P of this head: (Q K^T) masked to j <= t, scaled exp(G_t - G_j) ---
    {
      T *pf_out = (T *)a.Pf + ch * (int64_t)(64 * 64);
      frag pf[KS_C];
      const int t = 16 * tt + c;
      const float gt = Gr[t];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 16 * jt + 4 * g + e;
          const float pv = (j <= t) ? qk[jt][e] * gexp(gt - Gr[j]) : 0.f;
          const int sl = 4 * jt + e;
          pf[sl / 8][sl % 8] = (T)pv;
        }
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt)
        if (2 * kt <= tt)
          st_inter<NTS>(reinterpret_cast<frag *>(pf_out + (((int64_t)tt * KS_C + kt) * 64 + lane) * 8), pf[kt]);
    }
    lds_sync();  // the q rows (first head) or the previous head's T are consumed
    // ---- A = strictly-lower(beta_t exp(G_t - G_j) k_t.k_j) ------------------
    {
      float Gt[4], Bt[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Gt[e] = Gr[16 * it + 4 * g + e];
        Bt[e] = Br[16 * it + 4 * g + e];
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        const int j = 16 * jt + c;
        const float Gj = Gr[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * it + 4 * g + e;
          AT[t][j] = (j < t) ? Bt[e] * gexp(Gt[e] - Gj) * kk[jt][e] : 0.f;
        }
      }
    }
    lds_sync();
    // ---- T diagonal blocks (forward substitution, lane c = column c) --------
    {
      const int bw = wave;
      float tc[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float sacc = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) sacc = fmaf(-AT[16 * bw + i][16 * bw + m], tc[m], sacc);
        tc[i] = (i < c) ? 0.f : sacc;
      }
      if (g == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) AT[16 * bw + i][16 * bw + c] = tc[i];
      }
    }
    lds_sync();
    // ---- off-diagonal blocks, one row block at a time ----------------------
#pragma unroll
    for (int bi = 1; bi < 4; ++bi) {
      const int bj = wave;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      if (bj < bi) {
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        for (int m = bj; m < bi; ++m) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            x = Mfma<float>::mma(AT[16 * bi + c][16 * m + 4 * kt + g],
                                 AT[16 * m + 4 * kt + g][16 * bj + c], x);
        }
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          y = Mfma<float>::mma(AT[16 * bi + c][16 * bi + 4 * g + kt], x[kt], y);
      }
      lds_sync();
      if (bj < bi) {
#pragma unroll
        for (int e = 0; e < 4; ++e) AT[16 * bi + 4 * g + e][16 * bj + c] = -y[e];
      }
      lds_sync();
    }
    // ---- -T diag(beta) (rows 16 w + c, columns in pi order) and row scales --
    {
      const int w = wave;
      T *tf = (T *)a.Wf + ch * (int64_t)(64 * 64) + (int64_t)w * KS_C * 64 * 8;
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) {
        if (kt > 0 && w < 2) continue;  // above the diagonal: zero, not stored
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * kt + 16 * (e >> 2) + 4 * g + (e & 3);
          y[e] = -AT[16 * w + c][j] * Br[j];
        }
        st_inter<NTS>(reinterpret_cast<frag *>(tf + ((int64_t)kt * 64 + lane) * 8), M::pack(y));
      }
      if (wave == 0) {
        const float inv = sm.inv[lane], gt = Gr[lane];
        float *bw = a.Bw + ch * 128;
        bw[lane] = gexp(gt) * inv;
        bw[64 + lane] = gexp(Gr[63] - gt) * inv;
      }
    }
  }
}

template <typename T, int D, bool NTS>
static hipError_t launch_intra_tform_shared(const Args &a, hipStream_t s) {
  const size_t smem = sizeof(IntraSmemS<T, D>);
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = set_dynamic_lds((const void *)intra_tform_shared_kernel<T, D, NTS>, (int)smem, lds_set);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = a.cap * a.hk;
  if (blocks == 0) return hipSuccess;
  intra_tform_shared_kernel<T, D, NTS><<<dim3((unsigned)blocks), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D, bool NTS, bool SHK, bool TF = false>
static hipError_t launch_intra_h_nt(const Args &a, hipStream_t s) {
  const size_t smem = sizeof(IntraSmemB<T, D>);
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = set_dynamic_lds((const void *)intra_kernel_h<T, D, NTS, SHK, TF>, (int)smem, lds_set);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = a.cap * a.H;
  if (blocks == 0) return hipSuccess;
  intra_kernel_h<T, D, NTS, SHK, TF><<<dim3((unsigned)blocks), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_intra_h(const Args &a, hipStream_t s) {
  // T form (four-tile state pass, D = 128): K^T is not stored, so sab heads
  // sharing k heads need no variant of their own
  if constexpr (D == 128) {
    // q and k heads both shared by 2 .. 4 sab heads: one workgroup per q/k head
    const int R = a.H / a.hk;
    if (a.tform && R >= 2 && R <= 4 && a.hq == a.hk)
      return a.nt_stores ? launch_intra_tform_shared<T, D, true>(a, s)
                         : launch_intra_tform_shared<T, D, false>(a, s);
    if (a.tform)
      return a.nt_stores ? launch_intra_h_nt<T, D, true, false, true>(a, s)
                         : launch_intra_h_nt<T, D, false, false, true>(a, s);
  } else {
    if (a.tform) return hipErrorInvalidValue;
  }
  // SHK: the sab heads share k heads, whose normalised K^T is stored once
  if (a.H != a.hk)
    return a.nt_stores ? launch_intra_h_nt<T, D, true, true>(a, s)
                       : launch_intra_h_nt<T, D, false, true>(a, s);
  return a.nt_stores ? launch_intra_h_nt<T, D, true, false>(a, s)
                     : launch_intra_h_nt<T, D, false, false>(a, s);
}

hipError_t launch_intra(const Args &a, hipStream_t s) {
  if (a.dtype == GDN_BF16) {
    if (a.D == 128) return launch_intra_h<bf16, 128>(a, s);
    if (a.D == 64) return launch_intra_h<bf16, 64>(a, s);
    return launch_intra_h<bf16, 32>(a, s);
  }
  if (a.dtype == GDN_F16) {
    if (a.D == 128) return launch_intra_h<f16, 128>(a, s);
    if (a.D == 64) return launch_intra_h<f16, 64>(a, s);
    return launch_intra_h<f16, 32>(a, s);
  }
  if (a.D == 128) return launch_intra_t<float, 128>(a, s);
  if (a.D == 64) return launch_intra_t<float, 64>(a, s);
  return launch_intra_t<float, 32>(a, s);
}

}  // namespace gdn
