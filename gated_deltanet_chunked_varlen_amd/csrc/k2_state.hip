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
// register-reuse note in gdn_common.h).  Per chunk it also hands the
// chunk-start state and N to the output (stored for the fp32 output pass, or
// passed through LDS to the output waves of the fused 16-bit pass below),
// writes checkpoints (gitcode "FlashInfer GDN Prefill 完全指南", section
// "中间状态检查点") and, at the end, the final state into output_state (row
// state_indices[i] for a pool, section "状态池").
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

// Operands of one chunk for one 16-column tile, as loaded by one lane.
template <typename T, int D>
struct ChunkOps {
  typedef typename Mfma<T>::frag frag;
  static constexpr int NT = Geo<T, D>::NT, KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  frag w[4][KS_D];     // W rows (4 tiles), contraction over dk
  frag k[NT][KS_C];    // Ktilde^T rows (NT tiles), contraction over t
  T u[4][4];           // U in result layout
  float glog;          // G at the chunk's last row

  __device__ __forceinline__ void load(const Args &a, int64_t ch, int jv, int lane) {
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
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) u[it][r] = uf[((int64_t)it * 64 + lane) * 4 + r];
    glog = a.Gw[ch * kChunk + (kChunk - 1)];
  }
};

// Operands held in registers (ChunkOps) ...
template <typename T, int D>
struct RegOps {
  static constexpr bool kInterleave = false;
  const ChunkOps<T, D> &op;
  __device__ __forceinline__ typename Mfma<T>::frag w(int it, int kt) const { return op.w[it][kt]; }
  __device__ __forceinline__ typename Mfma<T>::frag k(int it, int kt) const { return op.k[it][kt]; }
  __device__ __forceinline__ f32x4 uvec(int it) const {
    return f32x4{to_f32(op.u[it][0]), to_f32(op.u[it][1]), to_f32(op.u[it][2]), to_f32(op.u[it][3])};
  }
  __device__ __forceinline__ float glog() const { return op.glog; }
};

// ... or read from an LDS slot laid out like the workspace blocks:
// [W fragments][Ktilde fragments][U tiles of the group][G_last].
template <typename T, int D, int NCW>
struct SlotGeo {
  static constexpr int E = sizeof(T);
  static constexpr int W_BYTES = 64 * D * E;
  static constexpr int U_TILE_BYTES = 4 * 64 * 4 * E;
  static constexpr int K_OFF = W_BYTES;
  static constexpr int U_OFF = 2 * W_BYTES;
  static constexpr int G_OFF = U_OFF + NCW * U_TILE_BYTES;
  static constexpr int BYTES = (G_OFF + 4 + 15) / 16 * 16;
  static constexpr int NV_W = W_BYTES / (64 * 16);        // 16-byte loads per lane
  static constexpr int NV_U = NCW * U_TILE_BYTES / (64 * 16);
  static constexpr int NV = 2 * NV_W + NV_U;
};

template <typename T, int D, int NCW>
struct LdsOps {
  static constexpr bool kInterleave = true;
  typedef typename Mfma<T>::frag frag;
  static constexpr int KPL = Mfma<T>::KPL, KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  const unsigned char *slot;
  int lane, cw;
  __device__ __forceinline__ frag w(int it, int kt) const {
    return *reinterpret_cast<const frag *>(slot + (((it * KS_D + kt) * 64 + lane) * KPL) * sizeof(T));
  }
  __device__ __forceinline__ frag k(int it, int kt) const {
    return *reinterpret_cast<const frag *>(slot + SlotGeo<T, D, NCW>::K_OFF +
                                           (((it * KS_C + kt) * 64 + lane) * KPL) * sizeof(T));
  }
  __device__ __forceinline__ f32x4 uvec(int it) const {
    const T *up = reinterpret_cast<const T *>(slot + SlotGeo<T, D, NCW>::U_OFF) +
                  ((cw * 4 + it) * 64 + lane) * 4;
    return f32x4{to_f32(up[0]), to_f32(up[1]), to_f32(up[2]), to_f32(up[3])};
  }
  __device__ __forceinline__ float glog() const {
    return *reinterpret_cast<const float *>(slot + SlotGeo<T, D, NCW>::G_OFF);
  }
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
  float accf[16];
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

template <typename St, int D>
__device__ __forceinline__ void write_state_t(St *p, const int64_t str[4], int64_t row, int h,
                                              int vcol, int g, const float (&S)[D / 16][4]) {
  const int64_t base = row * str[0] + (int64_t)h * str[1] + (int64_t)vcol * str[2];
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
  else write_state_t<_Float16, D>((_Float16 *)base_ptr, str, row, h, vcol, g, S);
}

template <typename St, int D>
__device__ __forceinline__ void read_state_t(const St *p, const int64_t str[4], int64_t row, int h,
                                             int vcol, int g, float (&S)[D / 16][4]) {
  const int64_t base = row * str[0] + (int64_t)h * str[1] + (int64_t)vcol * str[2];
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
    else read_state_t<_Float16, D>((const _Float16 *)a.init, a.init_str, row, h, vcol, g, S);
  } else {
#pragma unroll
    for (int it = 0; it < D / 16; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[it][r] = 0.f;
  }
}

// Operands are double-buffered in registers where they fit (bf16, or fp32 up
// to D = 64): the loads of chunk c+1 are issued before chunk c's products.
template <typename T, int D>
struct Prefetch { static constexpr bool value = sizeof(T) == 2 || D <= 64; };

// Register-pipelined variant: one wave64 per 16-column tile, operands of
// chunk c+1 loaded into registers while chunk c computes.  Used for fp32.
template <typename T, int D>
__global__ void __launch_bounds__(64) state_kernel(Args a) {
  constexpr int NT = D / 16;
  const int b = blockIdx.x;
  const int jv = (b >> 3) % NT;
  const int u = (b / (8 * NT)) * 8 + (b & 7);
  const int H = a.H;
  if (u >= a.N * H) return;
  const int seq = u / H, h = u % H;
  const int lane = threadIdx.x, g = lane >> 4, c = lane & 15;
  const int vcol = 16 * jv + c;

  int f0, nc, len;
  seq_geometry(a, seq, lane, f0, nc, len);

  int64_t row = seq;
  bool row_ok = true;
  if (a.sidx) {
    row = ld_index(a.sidx, a.sidx_type, seq);
    row_ok = row >= 0 && row < a.pool_rows;
  }

  // S[it][r] = S[16 it + 4g + r][vcol]   (keys x values)
  float S[NT][4];
  read_state<D>(a, row_ok, row, h, vcol, g, S);

  const int64_t ck_base = a.ck_every > 0 ? ld_index(a.ck_cs, a.ck_cs_type, seq) : 0;
  auto checkpoint = [&](int cc) {
    if (a.ck_every > 0) {
      const int done = (cc + 1) * kChunk;
      if (done <= len && done % a.ck_every == 0) {
        const int64_t crow = ck_base + done / a.ck_every - 1;
        if (crow >= 0 && crow < a.ck_rows)
          write_state<T, D>(a.ck, a.ck_dtype, a.ck_str, crow, h, vcol, g, S);
      }
    }
  };
  const int64_t ch0 = ws_index(f0, h, a.cap);
  if (Prefetch<T, D>::value) {
    ChunkOps<T, D> op0, op1;
    if (nc > 0) op0.load(a, ch0, jv, lane);
    int cc = 0;
    for (; cc + 1 < nc; cc += 2) {
      op1.load(a, ch0 + (int64_t)(cc + 1), jv, lane);
      chunk_step<T, D>(a, RegOps<T, D>{op0}, S, ch0 + (int64_t)cc, jv, lane);
      checkpoint(cc);
      if (cc + 2 < nc) op0.load(a, ch0 + (int64_t)(cc + 2), jv, lane);
      chunk_step<T, D>(a, RegOps<T, D>{op1}, S, ch0 + (int64_t)(cc + 1), jv, lane);
      checkpoint(cc + 1);
    }
    if (cc < nc) {
      chunk_step<T, D>(a, RegOps<T, D>{op0}, S, ch0 + (int64_t)cc, jv, lane);
      checkpoint(cc);
    }
  } else {
    for (int cc = 0; cc < nc; ++cc) {
      ChunkOps<T, D> op;
      op.load(a, ch0 + (int64_t)cc, jv, lane);
      chunk_step<T, D>(a, RegOps<T, D>{op}, S, ch0 + (int64_t)cc, jv, lane);
      checkpoint(cc);
    }
  }

  if (a.out_final && a.outst && row_ok)
    write_state<T, D>(a.outst, a.out_dtype, a.out_str, row, h, vcol, g, S);
}


// ===========================================================================
// Fused state and output pass (16-bit inputs).
//
// 0539edu "GDN与线性注意力GPU并行实现", section 3.3, splits a chunk's output
// into what it reads from its start state and what it wrote itself; the
// state pass holds the first (S in registers) and produces the second's
// operand (N), so the output can be formed there instead of in a separate
// pass that would read both back from memory:
//
//   O = scale * ( diag(exp(G)) Q S + P N ),   P = (Q K^T) masked, from K1
//
// A workgroup owns one 16-column tile of one (sequence, head):
//   wave 0      compute: the recurrence; per chunk it reads W / Ktilde / U
//               from LDS and leaves the chunk's start-state and N fragments
//               in an LDS buffer;
//   OUTW waves  output: one chunk behind, O^T = S^T (diag(exp G) Q)^T +
//               N^T P^T for the tile's 16 columns, split over token tiles,
//               four consecutive columns per lane and 8-byte stores (only
//               rows inside the sequence);
//   NLW waves   loaders, in teams of TEAM waves (team j owns chunks
//               c = j mod NLW / TEAM): per chunk they fetch W, Ktilde, the
//               tile's U (compute part, two-slot ring) and q fragments, P
//               fragments and the gate row (output part, three-slot ring),
//               and store them into LDS together.
// Step st (one LDS-only barrier each): loaders store chunk st, the compute
// wave works on chunk st - 1, the output wave on chunk st - 2.
// ===========================================================================
template <typename T, int D>
struct OutSlotGeo {
  static constexpr int Q_BYTES = 64 * D * 2;
  static constexpr int P_OFF = Q_BYTES;
  static constexpr int P_BYTES = 64 * 64 * 2;
  static constexpr int G_OFF = P_OFF + P_BYTES;
  static constexpr int BYTES = G_OFF + 64 * 4;
  static constexpr int NV_Q = Q_BYTES / (64 * 16);
  static constexpr int NV_P = P_BYTES / (64 * 16);
};

template <typename T, int D, int TEAM>
struct FusedLoader {
  using CS = SlotGeo<T, D, 1>;
  using OS = OutSlotGeo<T, D>;
  static constexpr int64_t BLK = Geo<T, D>::W_ELEMS * sizeof(T) / 16;   // u32x4 per 64 x D block
  static constexpr int64_t PBLK = 64 * 64 * sizeof(T) / 16;              // u32x4 per P block
  static constexpr int NV = CS::NV + OS::NV_Q + OS::NV_P;                // pieces per chunk
  static constexpr int PPW = (NV + TEAM - 1) / TEAM;
  u32x4 v[PPW];
  float gv;
  int64_t uoff;
  int lane, part;

  __device__ __forceinline__ void init(int jg, int ln, int pt) {
    uoff = (int64_t)jg * (CS::U_TILE_BYTES / 16);
    lane = ln;
    part = pt;
  }
  // piece i of a chunk: W, Ktilde, U tile (compute slot), q, P (output slot)
  __device__ __forceinline__ void issue(const Args &a, int64_t ch) {
    const u32x4 *__restrict__ wf = reinterpret_cast<const u32x4 *>(a.Wf) + ch * BLK + lane;
    const u32x4 *__restrict__ kf = reinterpret_cast<const u32x4 *>(a.Kf) + ch * BLK + lane;
    const u32x4 *__restrict__ uf = reinterpret_cast<const u32x4 *>(a.Uf) + ch * BLK + uoff + lane;
    const u32x4 *__restrict__ qf = reinterpret_cast<const u32x4 *>(a.Qf) + ch * BLK + lane;
    const u32x4 *__restrict__ pf = reinterpret_cast<const u32x4 *>(a.Pf) + ch * PBLK + lane;
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
      const int i = part + TEAM * m;
      if (NV % TEAM == 0 || i < NV) {
        const u32x4 *src;
        if (i < CS::NV_W) src = wf + (int64_t)i * 64;
        else if (i < 2 * CS::NV_W) src = kf + (int64_t)(i - CS::NV_W) * 64;
        else if (i < CS::NV) src = uf + (int64_t)(i - 2 * CS::NV_W) * 64;
        else if (i < CS::NV + OS::NV_Q) src = qf + (int64_t)(i - CS::NV) * 64;
        else src = pf + (int64_t)(i - CS::NV - OS::NV_Q) * 64;
        v[m] = *src;
      }
    }
    if (part == 0) gv = a.Gw[ch * kChunk + lane];
  }
  __device__ __forceinline__ void drop(unsigned char *cslot, unsigned char *oslot) const {
    u32x4 *cdst = reinterpret_cast<u32x4 *>(cslot) + lane;
    u32x4 *odst = reinterpret_cast<u32x4 *>(oslot) + lane;
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
      const int i = part + TEAM * m;
      if (NV % TEAM == 0 || i < NV) {
        if (i < CS::NV) cdst[i * 64] = v[m];
        else odst[(i - CS::NV) * 64] = v[m];
      }
    }
    if (part == 0) {
      reinterpret_cast<float *>(oslot + OS::G_OFF)[lane] = gv;
      if (lane == kChunk - 1) *reinterpret_cast<float *>(cslot + CS::G_OFF) = gv;
    }
  }
};

// The output of one chunk for one 16-column tile (output wave).
template <typename T, int D, int OUTW>
__device__ __forceinline__ void output_step(const Args &a, const unsigned char *oslot,
                                            const typename Mfma<T>::frag *xb, int jv,
                                            int64_t tok0, int rows, int h, int lane, int ow) {
  using M = Mfma<T>;
  typedef typename M::frag frag;
  using OS = OutSlotGeo<T, D>;
  constexpr int KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  const int g = lane >> 4, c = lane & 15;
  const frag *qf = reinterpret_cast<const frag *>(oslot);
  const frag *pf = reinterpret_cast<const frag *>(oslot + OS::P_OFF);
  const float *gs = reinterpret_cast<const float *>(oslot + OS::G_OFF);
  frag sf[KS_D], nf[KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt) sf[kt] = xb[kt * 64 + lane];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt) nf[kt] = xb[(KS_D + kt) * 64 + lane];
  T *out = (T *)a.out;
  const int H = a.H;
#pragma unroll
  for (int i = 0; i < 4 / OUTW; ++i) {
    // token tiles of output wave ow: all four, or {0, 3} / {1, 2} (equal work)
    const int tt = OUTW == 1 ? i : (i == 0 ? ow : 3 - ow);
    const int t = 16 * tt + c;  // this lane's output row
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt) acc = M::mma(sf[kt], qf[(tt * KS_D + kt) * 64 + lane], acc);
    const float gam = gexp(gs[t]);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= gam;
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt)
      if (kt * 2 <= tt)  // k-step's first token tile is not masked out
        acc = M::mma(nf[kt], pf[(tt * KS_C + kt) * 64 + lane], acc);
    // acc[r] = O[t][16 jv + 4g + r]
    if (t < rows) {
      typename M::half o4;
#pragma unroll
      for (int r = 0; r < 4; ++r) o4[r] = (T)(a.scale * acc[r]);
      *reinterpret_cast<typename M::half *>(out + ((tok0 + t) * H + h) * D + 16 * jv + 4 * g) = o4;
    }
  }
}

template <typename T, int D, int OUTW, int NLW, int TEAM>
__global__ void __launch_bounds__(64 * (1 + OUTW + NLW)) state_output_kernel(Args a) {
  constexpr int NT = D / 16;
  using CS = SlotGeo<T, D, 1>;
  using OS = OutSlotGeo<T, D>;
  typedef typename Mfma<T>::frag frag;
  constexpr int XB = Geo<T, D>::KS_D + Geo<T, D>::KS_C;  // fragments per chunk in xbuf
  __shared__ __align__(16) unsigned char cslots[2][CS::BYTES];
  __shared__ __align__(16) unsigned char oslots[3][OS::BYTES];
  __shared__ frag xbuf[2][XB * 64];

  const int b = blockIdx.x;
  const int jg = (b >> 3) % NT;
  const int u = (b / (8 * NT)) * 8 + (b & 7);
  const int H = a.H;
  if (u >= a.N * H) return;
  const int seq = u / H, h = u % H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;

  int f0, nc, len, sbos;
  seq_geometry(a, seq, lane, f0, nc, len, sbos);
  const int64_t ch0 = ws_index(f0, h, a.cap);

  if (wave == 0) {
    // ---------------- compute wave ------------------------------------------
    const int vcol = 16 * jg + c;
    int64_t row = seq;
    bool row_ok = true;
    if (a.sidx) {
      row = ld_index(a.sidx, a.sidx_type, seq);
      row_ok = row >= 0 && row < a.pool_rows;
    }
    float S[NT][4];
    read_state<D>(a, row_ok, row, h, vcol, g, S);
    const int64_t ck_base = a.ck_every > 0 ? ld_index(a.ck_cs, a.ck_cs_type, seq) : 0;
    for (int st = 0; st <= nc + 1; ++st) {
      lds_sync();
      if (st == 0 || st > nc) continue;
      const int cc = st - 1;
      const LdsOps<T, D, 1> op{cslots[cc & 1], lane, 0};
      chunk_step<T, D>(a, op, S, ch0 + (int64_t)cc, jg, lane, xbuf[cc & 1]);
      if (a.ck_every > 0) {
        const int done = (cc + 1) * kChunk;
        if (done <= len && done % a.ck_every == 0) {
          const int64_t crow = ck_base + done / a.ck_every - 1;
          if (crow >= 0 && crow < a.ck_rows)
            write_state<T, D>(a.ck, a.ck_dtype, a.ck_str, crow, h, vcol, g, S);
        }
      }
    }
    if (a.out_final && a.outst && row_ok)
      write_state<T, D>(a.outst, a.out_dtype, a.out_str, row, h, vcol, g, S);
  } else if (wave <= OUTW) {
    // ---------------- output waves: one chunk behind the compute wave --------
    for (int st = 0; st <= nc + 1; ++st) {
      lds_sync();
      if (st < 2) continue;
      const int oc = st - 2;
      output_step<T, D, OUTW>(a, oslots[oc % 3], xbuf[oc & 1], jg,
                              (int64_t)sbos + (int64_t)kChunk * oc, min(kChunk, len - kChunk * oc),
                              h, lane, wave - 1);
    }
  } else {
    // ---------------- loader waves ------------------------------------------
    constexpr int NTEAM = NLW / TEAM;
    static_assert(NLW % TEAM == 0, "loader waves split into whole teams");
    const int lw = wave - 1 - OUTW, team = lw / TEAM;
    FusedLoader<T, D, TEAM> ld;
    ld.init(jg, lane, lw % TEAM);
    if (team < nc) ld.issue(a, ch0 + (int64_t)team);
    for (int st = 0; st <= nc + 1; ++st) {
      lds_sync();
      if (st < nc && st % NTEAM == team) {
        ld.drop(cslots[st & 1], oslots[st % 3]);
        if (st + NTEAM < nc) ld.issue(a, ch0 + (int64_t)(st + NTEAM));
      }
    }
  }
}

#ifndef GDN_FUSED_OUTW
#define GDN_FUSED_OUTW 2
#endif
#ifndef GDN_FUSED_NLW
#define GDN_FUSED_NLW 5
#endif
#ifndef GDN_FUSED_TEAM
#define GDN_FUSED_TEAM 5
#endif

template <typename T, int D>
static hipError_t launch_state_output_t(const Args &a, hipStream_t s) {
  constexpr int NT = D / 16, OUTW = GDN_FUSED_OUTW, NLW = GDN_FUSED_NLW, TEAM = GDN_FUSED_TEAM;
  const int64_t units = (int64_t)a.N * a.H;
  if (units == 0) return hipSuccess;
  const int64_t blocks = ((units + 7) / 8) * 8 * NT;
  state_output_kernel<T, D, OUTW, NLW, TEAM>
      <<<dim3((unsigned)blocks), dim3(64 * (1 + OUTW + NLW)), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_state_output(const Args &a, hipStream_t s) {
  if (a.dtype == GDN_F16) {
    if (a.D == 128) return launch_state_output_t<f16, 128>(a, s);
    if (a.D == 64) return launch_state_output_t<f16, 64>(a, s);
    return launch_state_output_t<f16, 32>(a, s);
  }
  if (a.D == 128) return launch_state_output_t<bf16, 128>(a, s);
  if (a.D == 64) return launch_state_output_t<bf16, 64>(a, s);
  return launch_state_output_t<bf16, 32>(a, s);
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


// fp32 inputs (16-bit inputs take the fused state/output pass above)
hipError_t launch_state(const Args &a, hipStream_t s) {
  if (a.D == 128) return launch_state_t<float, 128>(a, s);
  if (a.D == 64) return launch_state_t<float, 64>(a, s);
  return launch_state_t<float, 32>(a, s);
}

}  // namespace gdn
