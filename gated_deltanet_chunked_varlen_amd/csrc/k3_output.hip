// k3_output.hip -- output pass for fp32 inputs.  (With 16-bit inputs the
// fused state/output pass in k2_state.hip forms the output instead.)
//
// Every token reads the state after its own update (weigao.cc "GDN 与 Chunked
// Prefill", section "块内 state 和块间 final state").  Inside a chunk that
// starts from state S with new values N (0539edu "GDN与线性注意力GPU并行实现",
// section 3.3: one product for what the chunk reads from its start state, one
// triangular-masked product for what it wrote itself):
//
//   O = scale * ( diag(exp(G)) Q S + (Q K^T .* M) N ),
//   M[t][j] = exp(G_t - G_j) for j <= t, else 0.
//
// One workgroup of four wave64s per (flat chunk, sab head).  q and k rows are
// staged in LDS (normalised when asked, with the same row normalisation as the
// intra-chunk pass).  Wave w first forms P's row tile w: P^T = K Q^T leaves
// each lane holding rows of P in the order the next product contracts over
// (pi order), matching the stored N; the tiles go to LDS.  Then wave w owns
// value tiles w*D/64 .. and produces all 64 rows of them, reading only its
// share of the chunk-start state and N.  The output tile is staged in LDS and
// leaves as whole 16-byte row segments; rows beyond the sequence end are not
// stored.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

template <typename T, int D>
struct OutSmem {
  static constexpr int PAD = 16 / sizeof(T);
  T Qs[64][D + PAD];
  union {
    T Ks[64][D + PAD];     // k rows, for P
    T Os[64][D + PAD];     // output tile staging, after P
  } ko;
  typename Mfma<T>::frag Pf[4][kChunk / (4 * Mfma<T>::KPL)][64];  // P rows as operand fragments
  float Gs[64];
};

template <typename T, int D>
__global__ void __launch_bounds__(256) output_kernel(Args a) {
  using M = Mfma<T>;
  using Ge = Geo<T, D>;
  typedef typename M::frag frag;
  constexpr int KPL = Ge::KPL, NT = Ge::NT, KS_D = Ge::KS_D, KS_C = Ge::KS_C;
  constexpr int TPW = (NT + 3) / 4;  // value tiles per wave
  extern __shared__ __align__(16) unsigned char smem_raw[];
  OutSmem<T, D> &sm = *reinterpret_cast<OutSmem<T, D> *>(smem_raw);

  const int H = a.H;
  const int f = (int)(blockIdx.x / H), h = (int)(blockIdx.x % H);
  const int64_t ch = ws_index(f, h, a.cap);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tb, len;
  chunk_geometry(a, f, lane, false, tb, len);
  if (len <= 0) return;
  const int64_t bos = tb;
  const int g = lane >> 4, c = lane & 15;

  // this wave's value tiles: chunk-start state and new-value fragments,
  // issued first so their latency overlaps the q/k staging
  const T *hf = (const T *)a.Hf + ch * Ge::H_ELEMS;
  const T *nfp = (const T *)a.Nf + ch * Ge::W_ELEMS;
  frag hfr[TPW][KS_D], nfr[TPW][KS_C];
#pragma unroll
  for (int x = 0; x < TPW; ++x) {
    const int jv = wave * TPW + x;
    if (jv < NT) {
#pragma unroll
      for (int kt = 0; kt < KS_D; ++kt)
        hfr[x][kt] = *reinterpret_cast<const frag *>(hf + (((int64_t)jv * KS_D + kt) * 64 + lane) * KPL);
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt)
        nfr[x][kt] = *reinterpret_cast<const frag *>(nfp + (((int64_t)jv * KS_C + kt) * 64 + lane) * KPL);
    }
  }

  {
    const int t = tid >> 2, p = tid & 3;
    const bool valid = t < len;
    const int qh = h / (H / a.hq), kh = h / (H / a.hk);
    float xq[D / 4], xk[D / 4];
    if (valid) {
      load_row_part<T, D>((const T *)a.q + ((bos + t) * a.hq + qh) * D, p, xq);
      load_row_part<T, D>((const T *)a.k + ((bos + t) * a.hk + kh) * D, p, xk);
    } else {
#pragma unroll
      for (int e = 0; e < D / 4; ++e) xq[e] = xk[e] = 0.f;
    }
    float iq = 1.f, ik = 1.f;
    if (a.l2norm) {
      iq = row_inv_norm<D>(xq);
      ik = row_inv_norm<D>(xk);
    }
#pragma unroll
    for (int e = 0; e < D / 4; ++e) {
      sm.Qs[t][row_part_idx(p, e)] = from_f32<T>(xq[e] * iq);
      sm.ko.Ks[t][row_part_idx(p, e)] = from_f32<T>(xk[e] * ik);
    }
    if (tid < 64) sm.Gs[tid] = a.Gw[ch * kChunk + tid];
  }
  lds_sync();

  // ---- P row tile tt = wave: P^T = K Q^T leaves P rows in operand order ---
  {
    const int tt = wave;
    frag pf[KS_C];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (jt <= tt) {
#pragma unroll
        for (int kt = 0; kt < KS_D; ++kt) {
          const int k0 = kt * 4 * KPL + g * KPL;
          const frag fa = *reinterpret_cast<const frag *>(&sm.ko.Ks[16 * jt + c][k0]);
          const frag fb = *reinterpret_cast<const frag *>(&sm.Qs[16 * tt + c][k0]);
          acc = M::mma(fa, fb, acc);
        }
      }
      // acc[r] = P[t = 16tt + c][j = 16jt + 4g + r]
      const int t = 16 * tt + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jt + 4 * g + r;
        const float pv = (j <= t) ? acc[r] * gexp(sm.Gs[t] - sm.Gs[j]) : 0.f;
        const int s = 4 * jt + r;
        M::set(pf[s / KPL], s % KPL, pv);
      }
    }
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) sm.Pf[tt][kt][lane] = pf[kt];
  }
  lds_sync();

  // ---- O = scale (diag(exp G) Q S + P N) for this wave's value tiles -------
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    frag qf[KS_D];
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
      for (int e = 0; e < KPL; ++e)
        M::set(qf[kt], e, to_f32(sm.Qs[16 * tt + c][pi_idx(g, kt * KPL + e)]));
    float gam[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) gam[r] = gexp(sm.Gs[16 * tt + 4 * g + r]);
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
      const int jv = wave * TPW + x;
      if (jv >= NT) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < KS_D; ++kt) acc = M::mma(qf[kt], hfr[x][kt], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= gam[r];
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt)
        if ((kt * KPL) / 4 <= tt)  // k-step's first token tile is not masked out
          acc = M::mma(sm.Pf[tt][kt][lane], nfr[x][kt], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sm.ko.Os[16 * tt + 4 * g + r][16 * jv + c] = from_f32<T>(a.scale * acc[r]);
    }
  }
  lds_sync();

  // ---- coalesced store of the valid rows ----------------------------------
  constexpr int VEC = 16 / sizeof(T);           // elements per 16-byte store
  constexpr int PER_ROW = D / VEC;
  T *out = (T *)a.out;
  for (int i = tid; i < 64 * PER_ROW; i += 256) {
    const int t = i / PER_ROW, x = (i % PER_ROW) * VEC;
    if (t < len)
      *reinterpret_cast<u32x4 *>(out + ((bos + t) * H + h) * D + x) =
          *reinterpret_cast<const u32x4 *>(&sm.ko.Os[t][x]);
  }
}

template <typename T, int D>
static hipError_t launch_output_t(const Args &a, hipStream_t s) {
  const size_t smem = sizeof(OutSmem<T, D>);
  static std::atomic<uint64_t> lds_set{0};
  {
    const hipError_t e = set_dynamic_lds((const void *)output_kernel<T, D>, (int)smem, lds_set);
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = a.cap * a.H;
  if (blocks == 0) return hipSuccess;
  output_kernel<T, D><<<dim3((unsigned)blocks), dim3(256), smem, s>>>(a);
  return hipGetLastError();
}

// fp32 inputs (16-bit inputs form the output inside the fused state pass)
hipError_t launch_output(const Args &a, hipStream_t s) {
  if (a.D == 128) return launch_output_t<float, 128>(a, s);
  if (a.D == 64) return launch_output_t<float, 64>(a, s);
  return launch_output_t<float, 32>(a, s);
}

}  // namespace gdn
