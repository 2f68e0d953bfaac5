// gdn_common.h -- device-side building blocks shared by the GDN prefill
// kernels (gfx950 / CDNA4, wave64).
//
// Matrix products use the CDNA matrix cores:
//   bf16: v_mfma_f32_16x16x32_bf16  (A 16x32, B 32x16, C 16x16 fp32)
//   fp16: v_mfma_f32_16x16x32_f16   (same shapes)
//   fp32: v_mfma_f32_16x16x4_f32    (A 16x4,  B 4x16,  C 16x16 fp32)
// Lane l = 16*g + c (g = l / 16 in 0..3, c = l % 16).  With KPL contraction
// elements per lane per instruction (8 for bf16 / fp16, 1 for fp32):
//   A operand: lane holds A[c][KPL*g + e], e < KPL   (row c of the 16-row tile)
//   B operand: lane holds B[KPL*g + e][c]            (column c)
//   C result : lane holds C[4*g + r][c], r < 4
//
// Register reuse across a chain of products.  A 16-row result tile leaves
// rows 4g..4g+3 in lane group g.  If the next product contracts over those
// rows, visiting them in the order
//     pi(g, s) = 16*(s / 4) + 4*g + (s % 4)         (slot s of lane group g)
// makes the result registers, taken in slot order, exactly the next B
// operand (slot s = KPL*kt + e for k-step kt, element e).  The other operand
// must then be stored with its contraction index permuted by pi.  The
// workspace therefore holds operands "fragment-major": for a 16-row tile and
// k-step kt, the 64 lanes' KPL-element fragments are contiguous, so every
// operand load is one coalesced 64*KPL-element block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef _Float16 f16;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// 16-byte register vector; HIP's uint4 is a struct of unions that keeps
// arrays of it out of registers, this native vector type does not.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

constexpr int kChunk = 64;
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return (_Float16)x; }

// ---------------------------------------------------------------------------
// 8-bit float storage of states (OCP FP8: E4M3 with no infinities, max 448;
// E5M2, max 57344).  Only states are stored this way: a store rounds the fp32
// value to nearest, ties to even, and saturates at the largest finite
// magnitude (no scaling); a load widens exactly.  NaN stays NaN.
// ---------------------------------------------------------------------------
struct fp8e4m3 { unsigned char b; };
struct fp8e5m2 { unsigned char b; };

// Largest finite value of a format whose largest finite encoding is MAXBITS.
template <int MB, int BIAS, unsigned MAXBITS>
constexpr float fp8_max_finite() {
  float v = (float)((MAXBITS & ((1u << MB) - 1u)) | (1u << MB));
  for (int i = 0; i < (int)(MAXBITS >> MB) - BIAS - MB; ++i) v *= 2.f;
  return v;
}

template <int MB, int BIAS, unsigned MAXBITS>
__device__ __forceinline__ unsigned char f32_to_fp8(float x) {
  const unsigned u = __float_as_uint(x);
  const unsigned char sign = (unsigned char)((u >> 24) & 0x80u);
  if ((u & 0x7fffffffu) > 0x7f800000u) return sign | 0x7fu;  // NaN
  const float a = fabsf(x);
  if (a >= fp8_max_finite<MB, BIAS, MAXBITS>()) return sign | (unsigned char)MAXBITS;  // saturate
  if (a == 0.f) return sign;
  constexpr int EMIN = 1 - BIAS;                  // exponent of the smallest normal
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
  if (e < EMIN) e = EMIN;                          // below: the subnormal quantum
  // a in units of the quantum 2^(e - MB), rounded to nearest, ties to even
  unsigned m = (unsigned)rintf(ldexpf(a, MB - e));
  if (m >= (2u << MB)) {                           // rounding carried into the next binade
    m >>= 1;
    ++e;
  }
  unsigned bits = m < (1u << MB) ? m                                   // subnormal
                                 : ((unsigned)(e + BIAS) << MB) | (m - (1u << MB));
  if (bits > MAXBITS) bits = MAXBITS;
  return sign | (unsigned char)bits;
}

template <int MB, int BIAS>
__device__ __forceinline__ float fp8_to_f32(unsigned char b, bool e_all_ones_is_special) {
  const unsigned E = (b & 0x7fu) >> MB, M = b & ((1u << MB) - 1u);
  constexpr unsigned EMAX = 0x7fu >> MB;
  float v;
  if (E == EMAX && e_all_ones_is_special) v = M ? __builtin_nanf("") : __builtin_inff();
  else if (E == 0) v = ldexpf((float)M, 1 - BIAS - MB);
  else v = ldexpf((float)(M | (1u << MB)), (int)E - BIAS - MB);
  return (b & 0x80u) ? -v : v;
}

__device__ __forceinline__ float to_f32(fp8e4m3 x) {
  // E4M3 (no infinities): only S.1111.111 is NaN
  return (x.b & 0x7fu) == 0x7fu ? __builtin_nanf("") : fp8_to_f32<3, 7>(x.b, false);
}
__device__ __forceinline__ float to_f32(fp8e5m2 x) { return fp8_to_f32<2, 15>(x.b, true); }
template <> __device__ __forceinline__ fp8e4m3 from_f32<fp8e4m3>(float x) {
  return fp8e4m3{f32_to_fp8<3, 7, 0x7eu>(x)};
}
template <> __device__ __forceinline__ fp8e5m2 from_f32<fp8e5m2>(float x) {
  return fp8e5m2{f32_to_fp8<2, 15, 0x7bu>(x)};
}

// Matrix-core traits per compute type.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  typedef bf16x4 half;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void set(frag &f, int e, float x) { f[e] = (bf16)x; }
  static __device__ __forceinline__ float get(const frag &f, int e) { return (float)f[e]; }
  // KPL consecutive fp32 values -> one operand fragment (packed conversions)
  static __device__ __forceinline__ frag pack(const float *x) {
    const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    return __builtin_convertvector(v, bf16x8);
  }
};

template <> struct Mfma<f16> {
  static constexpr int KPL = 8;
  typedef f16x8 frag;
  typedef f16x4 half;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void set(frag &f, int e, float x) { f[e] = (f16)x; }
  static __device__ __forceinline__ float get(const frag &f, int e) { return (float)f[e]; }
  static __device__ __forceinline__ frag pack(const float *x) {
    const f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    return __builtin_convertvector(v, f16x8);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void set(frag &f, int, float x) { f = x; }
  static __device__ __forceinline__ float get(const frag &f, int) { return f; }
  static __device__ __forceinline__ frag pack(const float *x) { return x[0]; }
};

// ---------------------------------------------------------------------------
// Transposed LDS reads (ds_read_b64_tr_b16).  For a row-major bf16 matrix X in
// LDS, lane l = 16g + c passing the address of
//     X[r0(g) + c / 4][col0 + 4 (c % 4)]
// receives X[r0(g) + e][col0 + c] for e = 0..3: four consecutive rows of one
// column.  (Within each 16-lane group, result element e of lane c is element
// c % 4 of the 8 bytes that lane 4e + c / 4 addressed.)  Two such reads give
// the eight-row operand run of a bf16 matrix-core fragment, so matrices can
// stay row-major in LDS and still feed products that contract over rows.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

template <typename T>
__device__ __forceinline__ i16x4 lds_read_tr4(const T *p) {
  static_assert(sizeof(T) == 2, "16-bit elements");
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4 *)(p));
}

// Rows r0(g) .. r0(g) + 3 and r1(g) .. r1(g) + 3 of column col0 + c of a
// row-major 16-bit LDS matrix with leading dimension ld, as one operand
// fragment.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag lds_col_frag(const T *X, int ld, int r0,
                                                               int r1, int col0, int c) {
  const int rr = c >> 2, cc = col0 + 4 * (c & 3);
  const i16x4 lo = lds_read_tr4(X + (r0 + rr) * ld + cc);
  const i16x4 hi = lds_read_tr4(X + (r1 + rr) * ld + cc);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename Mfma<T>::frag, v);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every outstanding global load and store of the calling wave; this
// one waits for the wave's LDS accesses alone, so global loads issued ahead of
// time stay in flight across it.  Use it where the waves of a workgroup
// exchange data through LDS only.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Contraction index of slot s in lane group g (see the header comment).
__device__ __forceinline__ int pi_idx(int g, int s) {
  return 16 * (s >> 2) + 4 * g + (s & 3);
}

// ---------------------------------------------------------------------------
// Workspace geometry.  Everything per (flat chunk f, sab head h), stored
// head-major: ch = h * cap + f (cap = flat-chunk capacity), so the chunks of
// one head that the state pass walks through sit next to each other.
//   Wf : [ch][4 row tiles][D/(4K) ksteps][64][K]      -W, contraction dk in pi order
//   Kf : [ch][D/16 row tiles][64/(4K)][64][K]          Ktilde^T, contraction t in pi order
//   Uf : [ch][D/16 dv tiles][4 row tiles][64][4]       U in result layout
//   Gw : [ch][64] fp32                                 cumulative log gate
//   Hf : [ch][D/16 dv tiles][D/(4K)][64][K]            chunk-start state, dk in pi order
//   Nf : [ch][D/16 dv tiles][64/(4K)][64][K]           new values, t in pi order
// (K = KPL.)  Each block is 64*D elements except Gw (64) and Hf (D*D).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t ws_index(int f, int h, int64_t cap) {
  return (int64_t)h * cap + f;
}

template <typename T, int D> struct Geo {
  static constexpr int KPL = Mfma<T>::KPL;
  static constexpr int NT = D / 16;             // 16-wide tiles along D
  static constexpr int KS_D = D / (4 * KPL);     // k-steps contracting over D
  static constexpr int KS_C = kChunk / (4 * KPL);// k-steps contracting over a chunk
  static constexpr int64_t W_ELEMS = 64 * D;
  static constexpr int64_t H_ELEMS = (int64_t)D * D;
};

// ---------------------------------------------------------------------------
// Canonical row L2 normalisation.  Four cooperating lanes (lane ^ 1, lane ^ 2
// partners, i.e. lanes 4r..4r+3) share one row of D elements; lane part p owns
// the 8-element runs x with (x / 8) % 4 == p.  Sum of squares in fp32 in
// increasing x within a lane, then (p0 + p1) + (p2 + p3).  Every kernel that
// normalises q or k uses this, so all of them see bit-identical rows.
// ---------------------------------------------------------------------------
// Lane moves through the VALU's data-parallel-primitive (DPP) controls of
// gfx9 instead of a shuffle through LDS: CTRL is the control word, rows (16
// lanes) outside ROW_MASK and lanes whose source falls outside their row read
// 0.  Controls used: quad_perm [1,0,3,2] = 0xB1 and [2,3,0,1] = 0x4E,
// row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_or_zero_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum and prefix maximum of non-negative ints over the 64
// lanes of a wave (exact; 0 is the identity of both)
__device__ __forceinline__ int wave_prefix_sum_i(int x) {
  x += dpp_or_zero_i<0x111>(x);
  x += dpp_or_zero_i<0x112>(x);
  x += dpp_or_zero_i<0x114>(x);
  x += dpp_or_zero_i<0x118>(x);
  x += dpp_or_zero_i<0x142, 0xA>(x);
  x += dpp_or_zero_i<0x143, 0xC>(x);
  return x;
}
__device__ __forceinline__ int wave_prefix_max_nonneg(int x) {
  x = max(x, dpp_or_zero_i<0x111>(x));
  x = max(x, dpp_or_zero_i<0x112>(x));
  x = max(x, dpp_or_zero_i<0x114>(x));
  x = max(x, dpp_or_zero_i<0x118>(x));
  x = max(x, dpp_or_zero_i<0x142, 0xA>(x));
  x = max(x, dpp_or_zero_i<0x143, 0xC>(x));
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: steps of 1, 2, 4, 8
// within each row, then each row's total carried into the later rows.
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x += dpp_or_zero<0x111>(x);
  x += dpp_or_zero<0x112>(x);
  x += dpp_or_zero<0x114>(x);
  x += dpp_or_zero<0x118>(x);
  x += dpp_or_zero<0x142, 0xA>(x);  // lane 15 of rows 0, 2 into rows 1, 3
  x += dpp_or_zero<0x143, 0xC>(x);  // lane 31 into rows 2, 3
  return x;
}

template <int D>
__device__ __forceinline__ float row_inv_norm(const float (&x)[D / 4]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) s = fmaf(x[i], x[i], s);
  s += dpp_or_zero<0xB1>(s);  // lane parts p ^ 1
  s += dpp_or_zero<0x4E>(s);  // lane parts p ^ 2
  return 1.0f / sqrtf(s + kNormEps);
}

// Element index (within a row of D) of the i-th value owned by lane part p.
__device__ __forceinline__ int row_part_idx(int p, int i) {
  return 32 * (i >> 3) + 8 * p + (i & 7);
}

// Load a token row part for row-normalisation, as fp32.
template <typename Tin, int D>
__device__ __forceinline__ void load_row_part(const Tin *row, int p, float (&x)[D / 4]) {
#pragma unroll
  for (int i = 0; i < D / 4; i += 8) {
    const Tin *src = row + 32 * (i >> 3) + 8 * p;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i + e] = to_f32(src[e]);
  }
}

// 16-bit (bf16 / fp16) row part of lane part p (the runs of load_row_part),
// optionally normalised with row_inv_norm, rounded back to the input type:
// NV = D / 32 fragments of 8 elements, fragment i holding row elements
// 32 i + 8 p .. + 7.  The intra-chunk and output passes both use this, so they
// see the same k rows.  inv (optional) receives the factor applied: the
// row's inverse norm, or 1 without normalisation.
template <typename T, int D>
__device__ __forceinline__ void load_norm_row16(const T *row, int p, bool valid, bool l2norm,
                                                typename Mfma<T>::frag (&out)[D / 32],
                                                float *inv_out = nullptr) {
  typedef typename Mfma<T>::frag frag;
  constexpr int NV = D / 32;
  u32x4 raw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i)
    raw[i] = valid ? *reinterpret_cast<const u32x4 *>(row + 32 * i + 8 * p) : u32x4{0, 0, 0, 0};
  if (!l2norm) {
#pragma unroll
    for (int i = 0; i < NV; ++i) out[i] = __builtin_bit_cast(frag, raw[i]);
    if (inv_out) *inv_out = 1.f;
    return;
  }
  float x[D / 4];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const frag r8 = __builtin_bit_cast(frag, raw[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 * i + e] = (float)r8[e];
  }
  const float inv = row_inv_norm<D>(x);
  if (inv_out) *inv_out = inv;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const f32x8 y = {x[8 * i] * inv,     x[8 * i + 1] * inv, x[8 * i + 2] * inv,
                     x[8 * i + 3] * inv, x[8 * i + 4] * inv, x[8 * i + 5] * inv,
                     x[8 * i + 6] * inv, x[8 * i + 7] * inv};
    out[i] = __builtin_convertvector(y, frag);
  }
}

// ---------------------------------------------------------------------------
// Sequence geometry of a small batch straight from cu_seqlens, held by one
// wave: lane i <= N reads cu_seqlens[i].  The sanitisation is the chunk-index
// builder's: starts are the running maximum of cu_seqlens clamped to [0, T];
// sequence i has length start[i + 1] - start[i] and ceil(length / 64) chunks,
// numbered sequence-major.  Every lane of the wave must call it.
// ---------------------------------------------------------------------------
struct SeqLane {
  int64_t raw;   // cu_seqlens[lane] as given (lanes <= N)
  int bos;       // sanitised start of sequence `lane` (lanes <= N)
  int len;       // its length (lanes < N, else 0)
  int cc0, cc1;  // chunks before it / up to and including it
};

__device__ __forceinline__ int64_t load_index_any(const void *p, int type, int64_t i) {
  return type == 1 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

__device__ __forceinline__ SeqLane seq_lane(const void *cu, int cu_type, int N, int64_t T,
                                            int lane) {
  SeqLane s;
  int64_t x = 0;
  s.raw = 0;
  if (lane <= N) {
    s.raw = cu ? load_index_any(cu, cu_type, lane) : (lane == 0 ? 0 : T);
    x = s.raw < 0 ? 0 : (s.raw > T ? T : s.raw);
  }
  // running maximum and chunk counts by DPP lane moves (no LDS round trips)
  const int bos = wave_prefix_max_nonneg((int)x);
  const int nxt = __shfl_down(bos, 1);
  s.bos = bos;
  s.len = lane < N ? nxt - bos : 0;
  const int nch = (s.len + kChunk - 1) / kChunk;
  const int cc = wave_prefix_sum_i(nch);
  s.cc1 = cc;
  s.cc0 = cc - nch;
  return s;
}

// (first token, length) of flat chunk f from a SeqLane wave; length 0 when f
// is past the last chunk.  Wave-uniform results.
__device__ __forceinline__ void chunk_from_lanes(const SeqLane &s, int N, int f, int lane,
                                                 int &tok, int &len) {
  const unsigned long long m = __ballot(lane < N && s.cc0 <= f && f < s.cc1);
  tok = 0;
  len = 0;
  if (m) {
    const int seq = __ffsll((long long)m) - 1;
    const int b0 = __shfl(s.bos, seq), c0 = __shfl(s.cc0, seq), l0 = __shfl(s.len, seq);
    tok = b0 + kChunk * (f - c0);
    len = min(kChunk, b0 + l0 - tok);
  }
}

// fp32 exp of a (non-positive) log-gate difference.
__device__ __forceinline__ float gexp(float x) { return __expf(x); }

// Generic state element access for the three state dtypes.
__device__ __forceinline__ float load_state_elem(const void *base, int dtype, int64_t off) {
  if (dtype == 0) return ((const float *)base)[off];
  if (dtype == 1) return (float)((const bf16 *)base)[off];
  return (float)((const _Float16 *)base)[off];
}
__device__ __forceinline__ void store_state_elem(void *base, int dtype, int64_t off, float x) {
  if (dtype == 0) ((float *)base)[off] = x;
  else if (dtype == 1) ((bf16 *)base)[off] = (bf16)x;
  else ((_Float16 *)base)[off] = (_Float16)x;
}

}  // namespace gdn
