// k5_cp.hip -- context parallelism within the GPU: segment transitions and
// the serial fix-up of segment start states.
//
// gitcode "FlashInfer GDN Prefill 完全指南", section "Cake GDN CP 后端"
// ("四阶段执行流程"): T precompute, then M/N precompute at the CP chunk
// boundaries, then a fix-up that makes the boundary states consistent, then
// the CP prefill proper.  0539edu "GDN与线性注意力GPU并行实现", sections 2.1
// and 2.2: the state update is affine in the state, S_c = A_c S_{c-1} + B_c,
// and such affine maps compose associatively, so a segment of chunks acts on
// its start state as one pair (M, S_local).
//
// With the chunk's W, Ktilde, U from the intra-chunk pass (S is keys x
// values; the workspace holds -W):
//
//   S_c = (exp(G_last) I - Ktilde^T W) S_{c-1} + Ktilde^T U = A_c S_{c-1} + B_c
//
// A segment of chunks c1..c2 maps its start state S0 to
//
//   S_end = M S0 + S_local,   M = A_c2 ... A_c1,
//
// where S_local is the segment's state from a zero start.  Column m of M is
// what the recurrence makes of the unit vector e_m with U = 0, so both halves
// run the ordinary chain over 2D columns: D columns of S_local (U tile, zero
// start) and D columns of M (no U, identity start).  Every segment but the
// last of its sequence is run this way, all at once (cp_transition_kernel).
// Then, per sequence, head and 16 value rows, the start states are chained
// serially over the segments (cp_fixup_kernel):
//
//   start_0 = initial state,   start_{p+1} = M_p start_p + S_local_p
//
// and the fused state/output pass runs every segment from its start state
// (state_output_kernel's context-parallel form in k2_state.hip).  Stored
// layouts: fp32 [N][nseg][H][D][D]; a state's row v holds S[:, v]; row m of
// a transition holds M[:, m].
#include "gdn_common.h"
#include "gdn_internal.h"
#include "gdn_state.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

namespace {

__device__ __forceinline__ float *cp_block(float *base, const Args &a, int seq, int seg, int h,
                                           int D) {
  return base + (((int64_t)seq * a.cp_nseg + seg) * a.H + h) * (int64_t)D * D;
}

}  // namespace

// One chunk for a pair of columns that share the chunk's operands: column
// tile jt of S_local (with the tile's U) and column tile jt of M (U = 0).
// The W and Ktilde fragments are read from the LDS slot once for both.
template <typename T, int D, typename Ops>
__device__ __forceinline__ void pair_step(const Ops &op, float (&S0)[D / 16][4],
                                          float (&S1)[D / 16][4]) {
  using M = Mfma<T>;
  using Ge = Geo<T, D>;
  typedef typename M::frag frag;
  constexpr int KPL = Ge::KPL, NT = Ge::NT, KS_D = Ge::KS_D, KS_C = Ge::KS_C;
  frag wv[4][KS_D];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
    for (int it = 0; it < 4; ++it) wv[it][kt] = op.w(it, kt);
  f32x4 acc0[4], acc1[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    acc0[it] = op.uvec(it);
    acc1[it] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float gl = gexp(op.glog());
  frag sb0[KS_D], sb1[KS_D];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt) {
    sb0[kt] = M::pack(&S0[0][0] + kt * KPL);
    sb1[kt] = M::pack(&S1[0][0] + kt * KPL);
  }
  // N = U + (-W) S for both columns
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      acc0[it] = M::mma(wv[it][kt], sb0[kt], acc0[it]);
      acc1[it] = M::mma(wv[it][kt], sb1[kt], acc1[it]);
    }
  float n0[16], n1[16];
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      n0[4 * it + r] = acc0[it][r];
      n1[4 * it + r] = acc1[it][r];
    }
  // where sab heads share a k head the slot holds the normalised K^T, and
  // the decay to the chunk's end scales N's rows (Ktilde^T N = K^T diag(.) N)
  if constexpr (Ops::kScaleN) {
    const int g = (op.lane >> 4);
    const float glast = op.glog();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 gv = op.grow4(16 * j + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = gexp(glast - gv[r]);
        n0[4 * j + r] *= f;
        n1[4 * j + r] *= f;
      }
    }
  }
  frag nf0[KS_C], nf1[KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt) {
    nf0[kt] = M::pack(n0 + kt * KPL);
    nf1[kt] = M::pack(n1 + kt * KPL);
  }
  // S' = exp(G_last) S + Ktilde^T N
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 s0 = {S0[it][0] * gl, S0[it][1] * gl, S0[it][2] * gl, S0[it][3] * gl};
    f32x4 s1 = {S1[it][0] * gl, S1[it][1] * gl, S1[it][2] * gl, S1[it][3] * gl};
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
      const frag kv = op.k(it, kt);
      s0 = M::mma(kv, nf0[kt], s0);
      s1 = M::mma(kv, nf1[kt], s1);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      S0[it][r] = s0[r];
      S1[it][r] = s1[r];
    }
  }
}

// Workgroup: column tiles 2q and 2q + 1 (q < D / 32) of one (sequence,
// segment, head), for S_local and for M.  Waves 0 and 1 compute (wave w:
// tile 2q + w of both, which read the same W and Ktilde fragments); waves 2
// and 3 load each chunk's W, Ktilde, the two U tiles and the gate row into a
// four-slot LDS ring with direct memory-to-LDS loads, two chunks ahead; wave
// 4 warms L2 two chunks further ahead when the intermediates live in HBM
// (a.warm, as in the fused pass).  Step st (one barrier each): the loaders
// start chunk st + 2 and wait for chunk st, the compute waves work on chunk
// st - 1.
constexpr int kCpTW = 2, kCpSlots = 4;

// L2 warm-up for the transition pass when the intermediates live in HBM: one
// 4-byte load per 128-byte line of a chunk's W and Ktilde blocks (the
// workgroups of one unit split them; they run on one XCD) and of the
// workgroup's own U tiles and gate row, into a junk LDS word.
template <typename T, int D>
struct TransWarm {
  static constexpr int NWG = D / 16 / kCpTW, LINE = 128;
  static constexpr int WL = Geo<T, D>::W_ELEMS * (int)sizeof(T) / LINE;  // lines per block
  static constexpr int SHARED = 2 * WL;
  static constexpr int UL = kCpTW * DmaSlotGeo<T, D>::U_TILE_BYTES / LINE;
  static constexpr int GL = 64 * 4 / LINE;
  static_assert(UL + GL <= 64, "one line per lane");
  __device__ __forceinline__ static void touch(const Args &a, int64_t ch, int h, int jw, int lane,
                                               unsigned char *junk) {
    const unsigned char *wf = (const unsigned char *)a.Wf + ch * (WL * LINE);
    const unsigned char *kf = (const unsigned char *)a.Kf + k_block(a, ch, h) * (WL * LINE);
#pragma unroll
    for (int l0 = 0; l0 < SHARED; l0 += NWG * 64) {
      const int l = min(l0 + jw + NWG * lane, SHARED - 1);
      dma4(l < WL ? wf + l * LINE : kf + (l - WL) * LINE, junk);
    }
    const unsigned char *uf = (const unsigned char *)a.Uf + ch * (WL * LINE) +
                              (int64_t)jw * kCpTW * DmaSlotGeo<T, D>::U_TILE_BYTES;
    const unsigned char *gw = (const unsigned char *)(a.Gw + ch * kChunk);
    const int l = min(lane, UL + GL - 1);
    dma4(l < UL ? uf + l * LINE : gw + (l - UL) * LINE, junk);
  }
};

template <typename T, int D, bool SHK>
__global__ void __launch_bounds__(320) cp_transition_kernel(Args a) {
  constexpr int NT = D / 16, NWG = NT / kCpTW, NLD = 2, NSLOT = kCpSlots, AHEAD = NSLOT - 2;
  using SG = DmaSlotGeo<T, D, kCpTW>;
  using LD = DmaLoader<T, D, NLD, kCpTW>;
  static_assert(AHEAD * LD::MIN_PER_PART <= 63, "vmcnt range");
  __shared__ __align__(16) unsigned char cslots[NSLOT][SG::BYTES];
  __shared__ __align__(16) unsigned char junk[256];

  const int b = blockIdx.x;
  const int jw = (b >> 3) % NWG;
  const int u = (b / (8 * NWG)) * 8 + (b & 7);
  const int H = a.H, NS = a.cp_nseg;
  if (u >= a.N * NS * H) return;
  const int h = u % H, sp = u / H, seg = sp % NS, seq = sp / NS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;

  int f0, nc, len;
  seq_geometry(a, seq, lane, f0, nc, len);
  const int c0 = seg * a.cp_seg;
  // the last segment's pair is never used, and segments past it are empty
  if (c0 + a.cp_seg >= nc) return;
  const int n = a.cp_seg;
  const int64_t ch0 = ws_index(f0 + c0, h, a.cap);

  if (wave < kCpTW) {
    const int jg = kCpTW * jw + wave;
    const int col = 16 * jg + c;
    // S0 = S_local tile (zero start), S1 = M tile (columns of the identity);
    // S[it][r] = X[16 it + 4 g + r][col]
    float S0[NT][4], S1[NT][4];
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        S0[it][r] = 0.f;
        S1[it][r] = (16 * it + 4 * g + r == col) ? 1.f : 0.f;
      }
    for (int st = 0; st <= n; ++st) {
      lds_sync();
      if (st == 0) continue;
      const int cc = st - 1;
      const DmaSlotOps<T, D, kCpTW, SHK> op{cslots[cc % NSLOT], lane, wave};
      pair_step<T, D>(op, S0, S1);
    }
    const int64_t str[4] = {0, 0, (int64_t)D, 1};
    write_state_t<float, D>(cp_block(a.cp_sloc, a, seq, seg, h, D), str, 0, 0, col, g, S0);
    // M in the fix-up's operand order: fix-up lane l = 16 (m % 4) + k % 16 of
    // wave k / 16 takes M[k][m] for m = 4 kk + m % 4 as float4 number kk / 4,
    // element kk % 4, and the 64 lanes' float4 number q are adjacent:
    // element M[k][m] at (((k / 16) * (D / 16) + m / 16) * 64 + l) * 4 + (m / 4) % 4
    float *mb = cp_block(a.cp_m, a, seq, seg, h, D);
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mb[((int64_t)(it * (D / 16) + (col >> 4)) * 64 + 16 * (col & 3) + 4 * g + r) * 4 +
           ((col >> 2) & 3)] = S1[it][r];
  } else if (wave == kCpTW + NLD) {
    const int ahead = a.warm;
    for (int cc = AHEAD; cc < AHEAD + ahead && cc < n; ++cc)
      TransWarm<T, D>::touch(a, ch0 + cc, h, jw, lane, junk);
    for (int st = 0; st <= n; ++st) {
      __builtin_amdgcn_s_barrier();
      if (ahead > 0 && st + AHEAD + ahead < n)
        TransWarm<T, D>::touch(a, ch0 + (int64_t)(st + AHEAD + ahead), h, jw, lane, junk);
    }
    wait_vm<0>();
  } else {
    const LD ld{(int64_t)kCpTW * jw * (SG::U_TILE_BYTES / 16), lane, wave - kCpTW,
                k_block(a, ch0, h) - ch0};
    for (int cc = 0; cc < AHEAD && cc < n; ++cc) ld.issue(a, ch0 + (int64_t)cc, cslots[cc]);
    for (int st = 0; st <= n; ++st) {
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      if (st + AHEAD < n) ld.issue(a, ch0 + (int64_t)(st + AHEAD), cslots[(st + AHEAD) % NSLOT]);
      // chunk st must have landed before the next barrier
      if (st < n) {
        const int newer = min(AHEAD, n - 1 - st);
        if (newer >= 2) wait_vm<2 * LD::MIN_PER_PART>();
        else if (newer == 1) wait_vm<LD::MIN_PER_PART>();
        else wait_vm<0>();
      }
    }
  }
}

// One workgroup per (sequence, head, 16 value rows): start_0 from the
// initial state (or zero), then start_{p+1} = M_p start_p + S_local_p for the
// sequence's segments in order.  In value-row form, with X_p[v][m] =
// start_p[m][v] (the stored row v): X_{p+1}[v][k] = sum_m X_p[v][m] Mrow_p[m][k]
// + Sloc_p[v][k], a 16 x D by D x D product per step on fp32 matrix cores,
// one 16-column output tile per wave.  A wave's share of the next segment's
// transition and local state is loaded into registers while the current
// product runs (both were written by the previous launch, so only X_p is on
// the serial path; the step barriers wait for LDS accesses only, so those
// loads stay in flight across them).  The 16 rows of X_p sit in LDS between
// steps (the product's result layout differs from its operand layout).
template <int D>
__global__ void __launch_bounds__(64 * (D / 16)) cp_fixup_kernel(Args a) {
  constexpr int NT = D / 16, KK = D / 4;
  const int b = blockIdx.x;
  const int jv = b % NT;
  const int u = b / NT;
  const int H = a.H;
  if (u >= a.N * H) return;
  const int h = u % H, seq = u / H;
  const int nt = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  __shared__ float X[16][D + 1];

  int f0, nc, len;
  seq_geometry(a, seq, lane, f0, nc, len);
  const int used = nc > 0 ? (nc + a.cp_seg - 1) / a.cp_seg : 1;

  // start_0: lane (g, c) of wave 0 reads row v = 16 jv + c, keys 16 it + 4 g + r
  if (nt == 0) {
    int64_t row = seq;
    bool row_ok = true;
    if (a.sidx) {
      row = ld_index(a.sidx, a.sidx_type, seq);
      row_ok = row >= 0 && row < a.pool_rows;
    }
    float S[NT][4];
    read_state<D>(a, row_ok, row, h, 16 * jv + c, g, S);
    const int64_t str[4] = {0, 0, (int64_t)D, 1};
    write_state_t<float, D>(cp_block(a.cp_start, a, seq, 0, h, D), str, 0, 0, 16 * jv + c, g, S);
#pragma unroll
    for (int it = 0; it < NT; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) X[c][16 * it + 4 * g + r] = S[it][r];
  }
  lds_sync();

  // this lane's operands of step p: B[g][c] = Mrow_p[4 kk + g][16 nt + c] for
  // every kk, and S_local_p at the result positions [16 jv + 4 g + r][16 nt + c];
  // a ring of PF steps in registers (written by the previous launch, the
  // blocks may sit in another XCD's L2 or in HBM: several steps of latency
  // are in flight at once)
  // (the transition pass stores M so that these are D / 16 float4 loads, each
  // over 1 KB that the wave's 64 lanes cover together).
  // Every step fetches (the last step's blocks again near the end), so the
  // compiler's wait before a use counts exactly the loads issued after it.
  constexpr int PF = 4;
  float bm[PF][KK], lc[PF][4];
  const int steps = used - 1;
  auto fetch = [&](int p, int buf) {
    p = min(p, steps - 1);
    const f32x4 *Mp = reinterpret_cast<const f32x4 *>(cp_block(a.cp_m, a, seq, p, h, D)) +
                      (int64_t)nt * (KK / 4) * 64 + lane;
    const float *Lp = cp_block(a.cp_sloc, a, seq, p, h, D) + (int64_t)(16 * jv + 4 * g) * D + 16 * nt + c;
#pragma unroll
    for (int q = 0; q < KK / 4; ++q) {
      const f32x4 x = Mp[q * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) bm[buf][4 * q + e] = x[e];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) lc[buf][r] = Lp[(int64_t)r * D];
  };
  auto step = [&](int p, int buf) {
    fetch(p + PF - 1, (buf + PF - 1) % PF);
    // four independent accumulation chains (kk mod 4), summed at the end
    f32x4 part[4];
    part[0] = f32x4{lc[buf][0], lc[buf][1], lc[buf][2], lc[buf][3]};
    part[1] = part[2] = part[3] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      part[kk & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(X[c][4 * kk + g], bm[buf][kk],
                                                          part[kk & 3], 0, 0, 0);
    f32x4 acc;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = (part[0][r] + part[1][r]) + (part[2][r] + part[3][r]);
    lds_sync();
    float *Sn = cp_block(a.cp_start, a, seq, p + 1, h, D);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      X[4 * g + r][16 * nt + c] = acc[r];
      Sn[(int64_t)(16 * jv + 4 * g + r) * D + 16 * nt + c] = acc[r];
    }
    lds_sync();
  };
  if (steps < 1) return;
#pragma unroll
  for (int i = 0; i < PF - 1; ++i) fetch(i, i);
  int p = 0;
  for (; p + PF <= steps; p += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) step(p + i, i);
  }
#pragma unroll
  for (int i = 0; i < PF - 1; ++i)
    if (p + i < steps) step(p + i, i);
}

hipError_t launch_cp_transition(const Args &a, hipStream_t s) {
  constexpr int D = 128, NWG = D / 16 / kCpTW;
  const int64_t units = (int64_t)a.N * a.cp_nseg * a.H;
  if (units == 0 || a.D != D) return units == 0 ? hipSuccess : hipErrorInvalidValue;
  const int64_t blocks = ((units + 7) / 8) * 8 * NWG;
  const dim3 grid((unsigned)blocks), block(320);
  const bool shk = a.H != a.hk;   // sab heads share k heads (GQA / GVA)
  if (a.dtype == GDN_F16) {
    if (shk) cp_transition_kernel<f16, D, true><<<grid, block, 0, s>>>(a);
    else cp_transition_kernel<f16, D, false><<<grid, block, 0, s>>>(a);
  } else {
    if (shk) cp_transition_kernel<bf16, D, true><<<grid, block, 0, s>>>(a);
    else cp_transition_kernel<bf16, D, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_cp_fixup(const Args &a, hipStream_t s) {
  constexpr int D = 128;
  const int64_t units = (int64_t)a.N * a.H;
  if (units == 0 || a.D != D) return units == 0 ? hipSuccess : hipErrorInvalidValue;
  cp_fixup_kernel<D><<<dim3((unsigned)(units * (D / 16))), dim3(64 * (D / 16)), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace gdn
