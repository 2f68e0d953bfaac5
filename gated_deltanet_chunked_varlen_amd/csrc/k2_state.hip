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
template <typename T, int D, typename Ops>
__device__ __forceinline__ void chunk_step(const Args &a, const Ops &op,
                                           float (&S)[D / 16][4], int64_t ch, int jv,
                                           int lane) {
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
  {
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
      *reinterpret_cast<frag *>(nfp + ((int64_t)kt * 64 + lane) * KPL) = nf[kt];
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


// Loader waves per workgroup of the bf16 state pass.
#ifndef GDN_STATE_NLW
#define GDN_STATE_NLW 6
#endif
// loader waves that store one chunk into LDS together
#ifndef GDN_STATE_TEAM
#define GDN_STATE_TEAM 3
#endif

// One chunk's operands split over the TEAM loader waves of a team: wave part p
// of the team holds the 16-byte pieces i = p (mod TEAM) of the chunk's LDS
// slot, so storing a chunk into LDS takes TEAM waves in parallel.
template <typename T, int D, int NCW, int TEAM>
struct TeamLoader {
  using SG = SlotGeo<T, D, NCW>;
  static constexpr int64_t BLK = Geo<T, D>::W_ELEMS * sizeof(T) / 16;  // u32x4 per block
  static constexpr int PPW = (SG::NV + TEAM - 1) / TEAM;              // pieces per wave
  u32x4 v[PPW];
  float glog;
  int64_t uoff;
  int lane, part;

  __device__ __forceinline__ void init(int jg, int ln, int pt) {
    uoff = (int64_t)jg * NCW * (SG::U_TILE_BYTES / 16);
    lane = ln;
    part = pt;
  }
  __device__ __forceinline__ void issue(const Args &a, int64_t ch) {
    const u32x4 *__restrict__ wf = reinterpret_cast<const u32x4 *>(a.Wf) + ch * BLK + lane;
    const u32x4 *__restrict__ kf = reinterpret_cast<const u32x4 *>(a.Kf) + ch * BLK + lane;
    const u32x4 *__restrict__ uf = reinterpret_cast<const u32x4 *>(a.Uf) + ch * BLK + uoff + lane;
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
      const int i = part + TEAM * m;
      if (SG::NV % TEAM == 0 || i < SG::NV) {
        const u32x4 *src = i < SG::NV_W ? wf + (int64_t)i * 64
                         : i < 2 * SG::NV_W ? kf + (int64_t)(i - SG::NV_W) * 64
                                            : uf + (int64_t)(i - 2 * SG::NV_W) * 64;
        v[m] = *src;
      }
    }
    if (part == 0) glog = a.Gw[ch * kChunk + (kChunk - 1)];
  }
  __device__ __forceinline__ void drop(unsigned char *slot) const {
    u32x4 *dst = reinterpret_cast<u32x4 *>(slot) + lane;
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
      const int i = part + TEAM * m;
      if (SG::NV % TEAM == 0 || i < SG::NV) dst[i * 64] = v[m];
    }
    if (part == 0 && lane == 0) *reinterpret_cast<float *>(slot + SG::G_OFF) = glog;
  }
};

// Producer/consumer variant (bf16).  A workgroup owns NCW adjacent 16-column
// tiles of one (sequence, head): NCW compute waves run the recurrence, NLW
// loader waves keep the operands of upcoming chunks in flight in their own
// registers.  Loader w owns chunks c = w (mod NLW): it issues chunk c's loads
// NLW steps ahead and drops the data into LDS slot c % 2 during step c, while
// the compute waves work on chunk c - 1 from the other slot.  One LDS-only
// barrier per step orders the two (a full barrier would also wait for the
// loads in flight and undo the look-ahead).  The compute waves share every
// W / Ktilde fragment they read.
template <typename T, int D, int NCW, int NLW>
__global__ void __launch_bounds__(64 * (NCW + NLW)) state_kernel_pipe(Args a) {
  constexpr int NT = D / 16;
  constexpr int NGRP = NT / NCW;
  using SG = SlotGeo<T, D, NCW>;
  __shared__ __align__(16) unsigned char slots[2][SG::BYTES];

  const int b = blockIdx.x;
  const int jg = (b >> 3) % NGRP;
  const int u = (b / (8 * NGRP)) * 8 + (b & 7);
  const int H = a.H;
  if (u >= a.N * H) return;
  const int seq = u / H, h = u % H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;

  int f0, nc, len;
  seq_geometry(a, seq, lane, f0, nc, len);
  const int64_t ch0 = ws_index(f0, h, a.cap);

  if (wave < NCW) {
    // ---------------- compute wave: tile jv -------------------------------
    const int jv = jg * NCW + wave;
    const int vcol = 16 * jv + c;
    int64_t row = seq;
    bool row_ok = true;
    if (a.sidx) {
      row = ld_index(a.sidx, a.sidx_type, seq);
      row_ok = row >= 0 && row < a.pool_rows;
    }
    float S[NT][4];
    read_state<D>(a, row_ok, row, h, vcol, g, S);
    const int64_t ck_base = a.ck_every > 0 ? ld_index(a.ck_cs, a.ck_cs_type, seq) : 0;
    for (int st = 0; st <= nc; ++st) {
      lds_sync();
      if (st == 0) continue;
      const int cc = st - 1;
      const LdsOps<T, D, NCW> op{slots[cc & 1], lane, wave};
      chunk_step<T, D>(a, op, S, ch0 + (int64_t)cc, jv, lane);
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
  } else {
    // ---------------- loader waves -----------------------------------------
    // NLW / TEAM teams; team j owns chunks c = j (mod NLW / TEAM) and its
    // TEAM waves load and store each of them together.  The loads stay in
    // flight across the LDS-only barriers, so they have NLW / TEAM steps to
    // arrive.
    constexpr int NTEAM = NLW / GDN_STATE_TEAM;
    static_assert(NLW % GDN_STATE_TEAM == 0, "loader waves split into whole teams");
    const int lw = wave - NCW, team = lw / GDN_STATE_TEAM;
    TeamLoader<T, D, NCW, GDN_STATE_TEAM> ld;
    ld.init(jg, lane, lw % GDN_STATE_TEAM);
    if (team < nc) ld.issue(a, ch0 + (int64_t)team);
    for (int st = 0; st <= nc; ++st) {
      lds_sync();
      if (st < nc && st % NTEAM == team) {
        ld.drop(slots[st & 1]);
        if (st + NTEAM < nc) ld.issue(a, ch0 + (int64_t)(st + NTEAM));
      }
    }
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


template <typename T, int D, int NCW, int NLW>
static hipError_t launch_state_pipe_t(const Args &a, hipStream_t s) {
  constexpr int NGRP = D / 16 / NCW;
  const int64_t units = (int64_t)a.N * a.H;
  if (units == 0) return hipSuccess;
  const int64_t blocks = ((units + 7) / 8) * 8 * NGRP;
  state_kernel_pipe<T, D, NCW, NLW><<<dim3((unsigned)blocks), dim3(64 * (NCW + NLW)), 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_state(const Args &a, hipStream_t s) {
  if (a.dtype == GDN_F16) {
    constexpr int NLW = GDN_STATE_NLW;
    const int64_t units = (int64_t)a.N * a.H;
    const bool wide = units * (a.D / 16) > (int64_t)a.num_cus;
    if (a.D == 128)
      return wide ? launch_state_pipe_t<f16, 128, 2, NLW>(a, s) : launch_state_pipe_t<f16, 128, 1, NLW>(a, s);
    if (a.D == 64)
      return wide ? launch_state_pipe_t<f16, 64, 2, NLW>(a, s) : launch_state_pipe_t<f16, 64, 1, NLW>(a, s);
    return wide ? launch_state_pipe_t<f16, 32, 2, NLW>(a, s) : launch_state_pipe_t<f16, 32, 1, NLW>(a, s);
  }
  if (a.dtype == GDN_BF16) {
    constexpr int NLW = GDN_STATE_NLW;
    // One compute wave (16 columns) per workgroup while the workgroups fit on
    // the CUs at once: that halves each CU's LDS traffic per column.  With
    // more (sequence, head) pairs than that, two compute waves per workgroup
    // halve the number of workgroups instead.
    const int64_t units = (int64_t)a.N * a.H;
    const bool wide = units * (a.D / 16) > (int64_t)a.num_cus;
    if (a.D == 128)
      return wide ? launch_state_pipe_t<bf16, 128, 2, NLW>(a, s) : launch_state_pipe_t<bf16, 128, 1, NLW>(a, s);
    if (a.D == 64)
      return wide ? launch_state_pipe_t<bf16, 64, 2, NLW>(a, s) : launch_state_pipe_t<bf16, 64, 1, NLW>(a, s);
    return wide ? launch_state_pipe_t<bf16, 32, 2, NLW>(a, s) : launch_state_pipe_t<bf16, 32, 1, NLW>(a, s);
  }
  if (a.D == 128) return launch_state_t<float, 128>(a, s);
  if (a.D == 64) return launch_state_t<float, 64>(a, s);
  return launch_state_t<float, 32>(a, s);
}

}  // namespace gdn
