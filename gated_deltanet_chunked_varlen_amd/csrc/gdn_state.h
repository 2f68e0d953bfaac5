// gdn_state.h -- device pieces of the chunk-level state recurrence shared by
// the state passes (k2_state.hip) and the context-parallel passes
// (k5_cp.hip): one chunk's operands, one chunk step of a 16-column state
// tile, and state reads and writes in every storage format.
#pragma once

#include "gdn_common.h"
#include "gdn_internal.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

__device__ __forceinline__ int64_t ld_index(const void *p, int type, int64_t i) {
  return type == GDN_I64 ? ((const int64_t *)p)[i] : (int64_t)((const int32_t *)p)[i];
}

// Operands of one chunk for one 16-column tile, as loaded by one lane.
template <typename T, int D>
struct ChunkOps {
  typedef typename Mfma<T>::frag frag;
  static constexpr int NT = Geo<T, D>::NT, KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  frag w[4][KS_D];     // W rows (4 tiles), contraction over dk
  frag k[NT][KS_C];    // Ktilde^T rows (NT tiles), contraction over t
  T u[4][4];           // U in result layout
  float glog;          // G at the chunk's last row

  // with_u false: U is not read (a transition column, whose U is zero)
  __device__ __forceinline__ void load(const Args &a, int64_t ch, int jv, int lane,
                                       bool with_u = true) {
    constexpr int KPL = Mfma<T>::KPL;
    const T *wf = (const T *)a.Wf + ch * Geo<T, D>::W_ELEMS;
    const T *kf = (const T *)a.Kf + ch * Geo<T, D>::W_ELEMS;
    const T *uf = (const T *)a.Uf + ch * Geo<T, D>::W_ELEMS + (int64_t)jv * 4 * 64 * 4;
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int kt = 0; kt < KS_D; ++kt)
        w[it][kt] = *reinterpret_cast<const frag *>(wf + (((int64_t)it * KS_D + kt) * 64 + lane) * KPL);
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt)
        k[it][kt] = *reinterpret_cast<const frag *>(kf + (((int64_t)it * KS_C + kt) * 64 + lane) * KPL);
    if (with_u) {
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) u[it][r] = uf[((int64_t)it * 64 + lane) * 4 + r];
    }
    glog = a.Gw[ch * kChunk + (kChunk - 1)];
  }
};

// Operands held in registers (ChunkOps) ...
template <typename T, int D>
struct RegOps {
  static constexpr bool kInterleave = false;
  static constexpr bool kScaleN = false;  // Kf holds Ktilde^T (fp32 inputs)
  const ChunkOps<T, D> &op;
  __device__ __forceinline__ typename Mfma<T>::frag w(int it, int kt) const { return op.w[it][kt]; }
  __device__ __forceinline__ typename Mfma<T>::frag k(int it, int kt) const { return op.k[it][kt]; }
  __device__ __forceinline__ f32x4 uvec(int it) const {
    return f32x4{to_f32(op.u[it][0]), to_f32(op.u[it][1]), to_f32(op.u[it][2]), to_f32(op.u[it][3])};
  }
  __device__ __forceinline__ float glog() const { return op.glog; }
};

// One chunk of the state recurrence for one lane's share of a 16-column tile.
// With xb non-null (the fused state/output pass) the chunk-start state and
// N fragments go to that LDS buffer instead of the workspace: KS_D state
// fragments, then KS_C new-value fragments, 64 lanes each.
template <typename T, int D, typename Ops>
__device__ __forceinline__ void chunk_step(const Args &a, const Ops &op,
                                           float (&S)[D / 16][4], int64_t ch, int jv,
                                           int lane,
                                           typename Mfma<T>::frag *xb = nullptr) {
  using M = Mfma<T>;
  using Ge = Geo<T, D>;
  typedef typename M::frag frag;
  constexpr int KPL = Ge::KPL, NT = Ge::NT, KS_D = Ge::KS_D, KS_C = Ge::KS_C;
  // The W fragments are read up front, so their reads are in flight together
  // instead of one ahead of each product; the Ktilde fragments are read
  // while the first product runs (one read per product issued).
  frag wv[4][KS_D], kv[NT][KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
    for (int it = 0; it < 4; ++it) wv[it][kt] = op.w(it, kt);
  f32x4 acc[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) acc[it] = op.uvec(it);
  const float gl = gexp(op.glog());
  // 16-bit inputs: the gate log-cumsum at this lane's 16 chunk rows (pi
  // order), read with the W fragments; their decay to the chunk's end is
  // formed while the first product runs (see below)
  // (only where K is shared between sab heads; otherwise the workspace holds
  // Ktilde^T itself)
  constexpr bool scale_n = Ops::kScaleN;
  f32x4 grows[4];
  if constexpr (scale_n) {
#pragma unroll
    for (int j = 0; j < 4; ++j) grows[j] = op.grow4(16 * j + 4 * (lane >> 4));
  }
  __builtin_amdgcn_sched_barrier(0);
  // the state as operand fragments (dk in pi order): slot s is S[s / 4][s % 4]
  const float *Sflat = &S[0][0];
  frag sb[KS_D];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt) sb[kt] = M::pack(Sflat + kt * KPL);
  // chunk-start state, stored for the output pass
  if (xb) {
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt) xb[kt * 64 + lane] = sb[kt];
  } else {
    T *hf = (T *)a.Hf + ch * Ge::H_ELEMS + (int64_t)jv * KS_D * 64 * KPL;
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt)
      *reinterpret_cast<frag *>(hf + ((int64_t)kt * 64 + lane) * KPL) = sb[kt];
  }
  // N = U + (-W) S      (the workspace holds -W)
  float accf[16], ndec[16];
  {
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
      for (int it = 0; it < 4; ++it) acc[it] = M::mma(wv[it][kt], sb[kt], acc[it]);
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) kv[it][kt] = op.k(it, kt);
    if (Ops::kInterleave) {
      // pair each product of the first GEMM with one Ktilde read
#pragma unroll
      for (int i = 0; i < 4 * KS_D; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
    }
    if constexpr (scale_n) {
      const float glast = op.glog();
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) ndec[4 * j + r] = gexp(glast - grows[j][r]);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[4 * it + r] = acc[it][r];
  }
  // new values as operand fragments (t in pi order), stored for the output pass
  frag nf[KS_C];
  {
    T *nfp = (T *)a.Nf + ch * Ge::W_ELEMS + (int64_t)jv * KS_C * 64 * KPL;
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
      nf[kt] = M::pack(accf + kt * KPL);
      if (xb) xb[(KS_D + kt) * 64 + lane] = nf[kt];
      else *reinterpret_cast<frag *>(nfp + ((int64_t)kt * 64 + lane) * KPL) = nf[kt];
    }
  }
  // Where sab heads share a k head (16-bit inputs), the workspace holds the
  // normalised K^T once per k head, and the chunk's decay to its end scales
  // N's rows instead: Ktilde^T N = K^T diag(exp(G_last - G)) N.
  if constexpr (scale_n) {
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) accf[s2] *= ndec[s2];
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) nf[kt] = M::pack(accf + kt * KPL);
  }
  // S' = exp(G_last) S + Ktilde^T N
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 s4 = {S[it][0] * gl, S[it][1] * gl, S[it][2] * gl, S[it][3] * gl};
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) s4 = M::mma(kv[it][kt], nf[kt], s4);
#pragma unroll
    for (int r = 0; r < 4; ++r) S[it][r] = s4[r];
  }
}

// A lane holds S[16 it + 4 g + r][vcol], r = 0..3: four consecutive k of
// row vcol of the stored [V, K] state.  With unit k stride and every such
// run aligned to its size (checked per call), each run moves as one vector
// access (16 bytes in fp32, 8 in 16 bits); otherwise element by element.
template <typename St>
__device__ __forceinline__ bool state_runs_aligned(const void *p, const int64_t str[4]) {
  constexpr int A = 4 * (int)sizeof(St);
  return str[3] == 1 && (uintptr_t)p % A == 0 && (str[0] * (int64_t)sizeof(St)) % A == 0 &&
         (str[1] * (int64_t)sizeof(St)) % A == 0 && (str[2] * (int64_t)sizeof(St)) % A == 0;
}

template <typename St, int D>
__device__ __forceinline__ void write_state_t(St *p, const int64_t str[4], int64_t row, int h,
                                              int vcol, int g, const float (&S)[D / 16][4]) {
  const int64_t base = row * str[0] + (int64_t)h * str[1] + (int64_t)vcol * str[2];
  if (state_runs_aligned<St>(p, str)) {
#pragma unroll
    for (int it = 0; it < D / 16; ++it) {
      St x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = from_f32<St>(S[it][r]);
      __builtin_memcpy(__builtin_assume_aligned(p + base + 16 * it + 4 * g, 4 * sizeof(St)), x,
                       sizeof(x));
    }
    return;
  }
#pragma unroll
  for (int it = 0; it < D / 16; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) p[base + (int64_t)(16 * it + 4 * g + r) * str[3]] = from_f32<St>(S[it][r]);
}

template <typename T, int D>
__device__ __forceinline__ void write_state(void *base_ptr, int dtype, const int64_t str[4],
                                         int64_t row, int h, int vcol, int g,
                                         const float (&S)[D / 16][4]) {
  if (dtype == GDN_F32) write_state_t<float, D>((float *)base_ptr, str, row, h, vcol, g, S);
  else if (dtype == GDN_BF16) write_state_t<bf16, D>((bf16 *)base_ptr, str, row, h, vcol, g, S);
  else if (dtype == GDN_F16) write_state_t<_Float16, D>((_Float16 *)base_ptr, str, row, h, vcol, g, S);
  else if (dtype == GDN_FP8_E4M3) write_state_t<fp8e4m3, D>((fp8e4m3 *)base_ptr, str, row, h, vcol, g, S);
  else write_state_t<fp8e5m2, D>((fp8e5m2 *)base_ptr, str, row, h, vcol, g, S);
}

template <typename St, int D>
__device__ __forceinline__ void read_state_t(const St *p, const int64_t str[4], int64_t row, int h,
                                             int vcol, int g, float (&S)[D / 16][4]) {
  const int64_t base = row * str[0] + (int64_t)h * str[1] + (int64_t)vcol * str[2];
  if (state_runs_aligned<St>(p, str)) {
#pragma unroll
    for (int it = 0; it < D / 16; ++it) {
      St x[4];
      __builtin_memcpy(x, __builtin_assume_aligned(p + base + 16 * it + 4 * g, 4 * sizeof(St)),
                       sizeof(x));
#pragma unroll
      for (int r = 0; r < 4; ++r) S[it][r] = to_f32(x[r]);
    }
    return;
  }
#pragma unroll
  for (int it = 0; it < D / 16; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[it][r] = to_f32(p[base + (int64_t)(16 * it + 4 * g + r) * str[3]]);
}

template <int D>
__device__ __forceinline__ void read_state(const Args &a, bool row_ok, int64_t row, int h,
                                           int vcol, int g, float (&S)[D / 16][4]) {
  if (a.init && row_ok) {
    if (a.init_dtype == GDN_F32) read_state_t<float, D>((const float *)a.init, a.init_str, row, h, vcol, g, S);
    else if (a.init_dtype == GDN_BF16) read_state_t<bf16, D>((const bf16 *)a.init, a.init_str, row, h, vcol, g, S);
    else if (a.init_dtype == GDN_F16) read_state_t<_Float16, D>((const _Float16 *)a.init, a.init_str, row, h, vcol, g, S);
    else if (a.init_dtype == GDN_FP8_E4M3) read_state_t<fp8e4m3, D>((const fp8e4m3 *)a.init, a.init_str, row, h, vcol, g, S);
    else read_state_t<fp8e5m2, D>((const fp8e5m2 *)a.init, a.init_str, row, h, vcol, g, S);
  } else {
#pragma unroll
    for (int it = 0; it < D / 16; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[it][r] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Direct memory-to-LDS operand loading (the fused state/output pass and the
// context-parallel transition pass).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// Direct loads into LDS: lane i's `bytes` bytes land at dst + bytes * i
// (dst is the same for the whole wave).  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16(const void *src, unsigned char *dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *src, unsigned char *dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void *)dst, 4, 0, 0);
}

// One LDS slot of the fused pass, laid out like the workspace blocks:
// [W fragments][Ktilde fragments][the tile's U][gate row (64 floats)].
// TW = 1 or 2 column tiles per workgroup: their U tiles sit side by side
// (adjacent in the workspace too).
template <typename T, int D, int TW = 1>
struct DmaSlotGeo {
  static constexpr int W_BYTES = 64 * D * (int)sizeof(T);
  static constexpr int U_TILE_BYTES = 4 * 64 * 4 * (int)sizeof(T);   // 64 rows x 16 columns
  static constexpr int K_OFF = W_BYTES, U_OFF = 2 * W_BYTES;
  static constexpr int G_OFF = U_OFF + TW * U_TILE_BYTES;
  static constexpr int BYTES = G_OFF + 64 * 4;
  static constexpr int NV_W = W_BYTES / 1024;                         // 1 KB pieces per block
  static constexpr int NP = 2 * NV_W + TW * U_TILE_BYTES / 1024;     // pieces (W, Ktilde, U)
};

// SCALE: the slot holds the normalised K^T of a k head shared by several sab
// heads (Ktilde^T otherwise), so the chunk step scales N's rows by the decay.
template <typename T, int D, int TW = 1, bool SCALE = false>
struct DmaSlotOps {
  static constexpr bool kInterleave = true;
  static constexpr bool kScaleN = SCALE;
  typedef typename Mfma<T>::frag frag;
  using SG = DmaSlotGeo<T, D, TW>;
  static constexpr int KPL = Mfma<T>::KPL, KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  const unsigned char *slot;
  int lane;
  int utile;  // which of the slot's U tiles
  __device__ __forceinline__ frag w(int it, int kt) const {
    return *reinterpret_cast<const frag *>(slot + (((it * KS_D + kt) * 64 + lane) * KPL) * sizeof(T));
  }
  __device__ __forceinline__ frag k(int it, int kt) const {
    return *reinterpret_cast<const frag *>(slot + SG::K_OFF + (((it * KS_C + kt) * 64 + lane) * KPL) * sizeof(T));
  }
  __device__ __forceinline__ f32x4 uvec(int it) const {
    const T *up = reinterpret_cast<const T *>(slot + SG::U_OFF + utile * SG::U_TILE_BYTES) +
                  (it * 64 + lane) * 4;
    return f32x4{to_f32(up[0]), to_f32(up[1]), to_f32(up[2]), to_f32(up[3])};
  }
  __device__ __forceinline__ float glog() const {
    return reinterpret_cast<const float *>(slot + SG::G_OFF)[kChunk - 1];
  }
  // gate log-cumsum at chunk rows p .. p + 3 (p a multiple of 4)
  __device__ __forceinline__ f32x4 grow4(int p) const {
    return *reinterpret_cast<const f32x4 *>(slot + SG::G_OFF + 4 * p);
  }
};

// Loader wave `part` of NLD: its share of a chunk's pieces (piece i goes to
// part i % NLD; the gate row, one 4-byte-per-lane load, to the last part).
template <typename T, int D, int NLD, int TW = 1>
struct DmaLoader {
  using SG = DmaSlotGeo<T, D, TW>;
  static constexpr int NV_W = SG::NV_W;
  static constexpr int64_t BLK = Geo<T, D>::W_ELEMS * sizeof(T) / 16;   // u32x4 per 64 x D block
  static constexpr int NPC = SG::NP + 1;                                 // loads per chunk
  static constexpr int PPW = (SG::NP + NLD - 1) / NLD;
  // fewest loads any part issues per chunk: vmcnt thresholds built from it
  // wait for at least the part's own older loads
  static constexpr int MIN_PER_PART = NPC / NLD;
  int64_t uoff;
  int lane, part;
  int64_t kdelta;  // k_block(ch) - ch: the k head's block for this sab head

  __device__ __forceinline__ void issue(const Args &a, int64_t ch, unsigned char *slot) const {
    const u32x4 *wf = reinterpret_cast<const u32x4 *>(a.Wf) + ch * BLK + lane;
    const u32x4 *kf = reinterpret_cast<const u32x4 *>(a.Kf) + (ch + kdelta) * BLK + lane;
    const u32x4 *uf = reinterpret_cast<const u32x4 *>(a.Uf) + ch * BLK + uoff + lane;
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
      const int i = part + NLD * m;
      if (i < SG::NP) {
        const u32x4 *src;
        if (i < NV_W) src = wf + (int64_t)i * 64;
        else if (i < 2 * NV_W) src = kf + (int64_t)(i - NV_W) * 64;
        else src = uf + (int64_t)(i - 2 * NV_W) * 64;
        dma16(src, slot + i * 1024);
      }
    }
    if (part == NLD - 1) dma4(a.Gw + ch * kChunk + lane, slot + SG::G_OFF);
  }
};

// vmcnt(n) for the loader's waits (n <= 63).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

}  // namespace gdn
