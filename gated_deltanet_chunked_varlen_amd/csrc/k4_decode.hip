// k4_decode.hip -- one decode step of the gated delta rule.
//
// weigao.cc "GDN 与 Chunked Prefill", section "Prefill 和 decode 的差异":
// after prefill, each decode step adds a single token per sequence, so the
// state update is applied once, with no chunked form:
//
//   S <- alpha (I - beta k k^T) S + beta k v^T,   o = scale * S^T q
//
// gitcode "FlashInfer GDN Prefill 完全指南", sections "GDN prefill" and
// "状态池": the decode side continues from the state prefill leaves, in the
// same [rows, H, V, K] layout and the same state_indices pool.
//
// Column v of S (stored contiguously over k as row v of the [V, K] state)
// depends on column v alone:
//   S'[:, v] = alpha S[:, v] + beta (v_v - alpha k . S[:, v]) k
//   o_v      = scale q . S'[:, v]
// so one wave64 owns 16 columns of one (sequence, head) and works on four at
// a time, 16 lanes per column, each lane holding D / 16 consecutive elements.
// Reads and writes of the state are whole 64-byte-or-larger row segments.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

// A lane's E consecutive elements of one state column (row v of the [V, K]
// layout).  With unit element stride and 16-byte alignment of every row
// segment (checked per call) they move as whole 16-byte (or E-element)
// vector accesses; otherwise element by element.
template <typename St, int E>
struct ColIO {
  static constexpr int BYTES = E * (int)sizeof(St);
  static constexpr int ALIGN = BYTES < 16 ? BYTES : 16;

  __device__ __forceinline__ static bool vec_ok(const void *base, const int64_t *str) {
    return str[3] == 1 && ((uintptr_t)base % ALIGN) == 0 &&
           (str[0] * (int64_t)sizeof(St)) % ALIGN == 0 &&
           (str[1] * (int64_t)sizeof(St)) % ALIGN == 0 &&
           (str[2] * (int64_t)sizeof(St)) % ALIGN == 0;
  }
  __device__ __forceinline__ static void load(const St *p, int64_t str3, bool vec, float (&s)[E]) {
    if (vec) {
      St t[E];
      __builtin_memcpy(t, __builtin_assume_aligned(p, ALIGN), BYTES);
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = to_f32(t[e]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] = to_f32(p[(int64_t)e * str3]);
    }
  }
  __device__ __forceinline__ static void store(St *p, int64_t str3, bool vec, const float (&s)[E]) {
    if (vec) {
      St t[E];
#pragma unroll
      for (int e = 0; e < E; ++e) t[e] = from_f32<St>(s[e]);
      __builtin_memcpy(__builtin_assume_aligned(p, ALIGN), t, BYTES);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) p[(int64_t)e * str3] = from_f32<St>(s[e]);
    }
  }
};

template <int E>
__device__ __forceinline__ bool state_vec_ok(const void *base, int dtype, const int64_t *str) {
  if (dtype == GDN_F32) return ColIO<float, E>::vec_ok(base, str);
  if (dtype == GDN_BF16) return ColIO<bf16, E>::vec_ok(base, str);
  if (dtype == GDN_F16) return ColIO<_Float16, E>::vec_ok(base, str);
  return ColIO<fp8e4m3, E>::vec_ok(base, str);   // both 8-bit types: 1-byte elements
}

template <int E>
__device__ __forceinline__ void load_state_col(const void *base, int dtype, const int64_t *str,
                                               int64_t off, bool vec, float (&s)[E]) {
  if (dtype == GDN_F32) ColIO<float, E>::load((const float *)base + off, str[3], vec, s);
  else if (dtype == GDN_BF16) ColIO<bf16, E>::load((const bf16 *)base + off, str[3], vec, s);
  else if (dtype == GDN_F16) ColIO<_Float16, E>::load((const _Float16 *)base + off, str[3], vec, s);
  else if (dtype == GDN_FP8_E4M3) ColIO<fp8e4m3, E>::load((const fp8e4m3 *)base + off, str[3], vec, s);
  else ColIO<fp8e5m2, E>::load((const fp8e5m2 *)base + off, str[3], vec, s);
}

template <int E>
__device__ __forceinline__ void store_state_col(void *base, int dtype, const int64_t *str,
                                                int64_t off, bool vec, const float (&s)[E]) {
  if (dtype == GDN_F32) ColIO<float, E>::store((float *)base + off, str[3], vec, s);
  else if (dtype == GDN_BF16) ColIO<bf16, E>::store((bf16 *)base + off, str[3], vec, s);
  else if (dtype == GDN_F16) ColIO<_Float16, E>::store((_Float16 *)base + off, str[3], vec, s);
  else if (dtype == GDN_FP8_E4M3) ColIO<fp8e4m3, E>::store((fp8e4m3 *)base + off, str[3], vec, s);
  else ColIO<fp8e5m2, E>::store((fp8e5m2 *)base + off, str[3], vec, s);
}

// Sum over the 16 lanes of a column group.
__device__ __forceinline__ float sum16(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 8);
  return x;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) decode_kernel(Args a) {
  constexpr int E = D / 16;   // elements of a column per lane
  constexpr int NG = D / 16;  // 16-column groups per (sequence, head)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = a.H, N = a.N;

  // the status word: workgroup 0 checks every state index and writes it
  if (blockIdx.x == 0 && a.status) {
    __shared__ unsigned bits_sh;
    if (threadIdx.x == 0) bits_sh = 0u;
    __syncthreads();
    if (a.sidx) {
      for (int i = threadIdx.x; i < N; i += blockDim.x) {
        const int64_t r = load_index_any(a.sidx, a.sidx_type, i);
        if (r < 0 || r >= a.pool_rows) atomicOr(&bits_sh, GDN_STATUS_STATE_INDEX);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) a.status[0] = (int32_t)bits_sh;
  }

  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;
  if (gw >= (int64_t)N * H * NG) return;
  const int grp = (int)(gw % NG);
  const int64_t sh = gw / NG;
  const int h = (int)(sh % H), seq = (int)(sh / H);

  int64_t row = seq;
  bool ok = true;
  if (a.sidx) {
    row = load_index_any(a.sidx, a.sidx_type, seq);
    ok = row >= 0 && row < a.pool_rows;
  }

  // q and k: lane position l16 holds elements l16 * E .. of the row
  const int l16 = lane & 15, cq = lane >> 4;
  const int qh = h / (H / a.hq), kh = h / (H / a.hk), vh = h / (H / a.hv);
  float q[E], k[E];
  {
    // rows are contiguous and D-element aligned, so a lane's E elements are
    // one aligned vector access
    const T *qp = (const T *)a.q + ((int64_t)seq * a.hq + qh) * D + l16 * E;
    const T *kp = (const T *)a.k + ((int64_t)seq * a.hk + kh) * D + l16 * E;
    ColIO<T, E>::load(qp, 1, true, q);
    ColIO<T, E>::load(kp, 1, true, k);
    if (a.l2norm) {
      // x / sqrt(sum x^2 + eps) in fp32, rounded back to the input type as
      // the prefill kernels do
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        sq = fmaf(q[e], q[e], sq);
        sk = fmaf(k[e], k[e], sk);
      }
      const float iq = 1.0f / sqrtf(sum16(sq) + kNormEps);
      const float ik = 1.0f / sqrtf(sum16(sk) + kNormEps);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        q[e] = to_f32(from_f32<T>(q[e] * iq));
        k[e] = to_f32(from_f32<T>(k[e] * ik));
      }
    }
  }
  const int64_t gi = (int64_t)seq * H + h;
  const float alpha = a.g ? a.g[gi] : 1.f;
  const float beta = a.beta ? a.beta[gi] : 1.f;
  const T *vp = (const T *)a.v + ((int64_t)seq * a.hv + vh) * D;
  T *op = (T *)a.out + ((int64_t)seq * H + h) * D;

  // all four columns' state loads first, so a wave has 4 x D / 16 elements
  // per lane in flight; then the updates; then the stores
  const bool vin = a.init && ok && state_vec_ok<E>(a.init, a.init_dtype, a.init_str);
  const bool vout = a.outst && state_vec_ok<E>(a.outst, a.out_dtype, a.out_str);
  float s[4][E], vv[4];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int v = grp * 16 + pass * 4 + cq;
    if (a.init && ok) {
      load_state_col<E>(a.init, a.init_dtype, a.init_str,
                        row * a.init_str[0] + (int64_t)h * a.init_str[1] +
                            (int64_t)v * a.init_str[2] + (int64_t)(l16 * E) * a.init_str[3],
                        vin, s[pass]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) s[pass][e] = 0.f;
    }
    vv[pass] = to_f32(vp[v]);
  }
  float o[4];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    float d1 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) d1 = fmaf(k[e], s[pass][e], d1);
    d1 = sum16(d1);
    const float coef = beta * (vv[pass] - alpha * d1);
    float ov = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      s[pass][e] = fmaf(alpha, s[pass][e], coef * k[e]);
      ov = fmaf(q[e], s[pass][e], ov);
    }
    o[pass] = sum16(ov);
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int v = grp * 16 + pass * 4 + cq;
    if (ok && a.out_final && a.outst)
      store_state_col<E>(a.outst, a.out_dtype, a.out_str,
                         row * a.out_str[0] + (int64_t)h * a.out_str[1] +
                             (int64_t)v * a.out_str[2] + (int64_t)(l16 * E) * a.out_str[3],
                         vout, s[pass]);
    if (l16 == 0) op[v] = from_f32<T>(a.scale * o[pass]);
  }
}

template <typename T, int D>
static hipError_t launch_decode_t(const Args &a, hipStream_t s) {
  const int64_t waves = (int64_t)a.N * a.H * (D / 16);
  const int64_t blocks = (waves + 3) / 4;
  decode_kernel<T, D><<<dim3((unsigned)(blocks > 0 ? blocks : 1)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode(const Args &a, hipStream_t s) {
  if (a.dtype == GDN_F16) {
    if (a.D == 128) return launch_decode_t<f16, 128>(a, s);
    if (a.D == 64) return launch_decode_t<f16, 64>(a, s);
    return launch_decode_t<f16, 32>(a, s);
  }
  if (a.dtype == GDN_BF16) {
    if (a.D == 128) return launch_decode_t<bf16, 128>(a, s);
    if (a.D == 64) return launch_decode_t<bf16, 64>(a, s);
    return launch_decode_t<bf16, 32>(a, s);
  }
  if (a.D == 128) return launch_decode_t<float, 128>(a, s);
  if (a.D == 64) return launch_decode_t<float, 64>(a, s);
  return launch_decode_t<float, 32>(a, s);
}

}  // namespace gdn
