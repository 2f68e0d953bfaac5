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
#include "gdn_state.h"
#include "../../include/gdn_prefill.h"

namespace gdn {

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
//               and the gate row from an LDS slot and leaves the chunk's
//               start-state and N fragments in an LDS buffer;
//   waves 3, 5  output, one chunk behind: O^T = S^T (diag(exp G) Q)^T +
//               N^T P^T for the tile's 16 columns, token tiles {0, 3} and
//               {1, 2} (equal work: the masked P blocks are skipped); each
//               fetches its own q and P fragments and gate values straight
//               into registers, two chunks ahead (a three-deep ring);
//   waves 1, 2  loaders: direct memory-to-LDS loads (no register or LDS
//               write instructions on the way) of W, Ktilde, the tile's U
//               and the gate row into a four-slot ring, two chunks ahead;
//   wave 4      L2 warm-up (when the intermediates live in HBM): touches
//               the lines of the chunk two ahead.
// When the intermediates live in HBM, waves 1 and 4 swap roles (below).
// Step st (one barrier each): the loaders start chunk st + 2 and wait for
// chunk st, the compute wave works on chunk st - 1, the output waves on
// chunk st - 2 and start fetching chunk st.  Larger batches give a
// workgroup two or four adjacent column tiles (FusedRoles below), which
// share the W / Ktilde and q / P loads; the context-parallel form runs the
// same pass over segments of sequences (k5_cp.hip).
// ===========================================================================
// L2 warm-up of a chunk ahead of the loaders and output waves: one 4-byte
// load per 128-byte line of everything the chunk's workgroups will read,
// sent into a junk LDS word (nothing waits on it).  The NT workgroups of a
// (sequence, head) share one XCD's L2 (consecutive ids map round-robin onto
// the 8 XCDs), so each touches every NT-th line of the shared W, Ktilde, q
// and P blocks, plus its own U tile and the gate row.
template <typename T, int D, int TW = 1>
struct L2Warm {
  static constexpr int NWG = D / 16 / TW;  // workgroups per (sequence, head)
  static constexpr int LINE = 128;
  static constexpr int WL = Geo<T, D>::W_ELEMS * (int)sizeof(T) / LINE;  // lines per 64 x D block
  static constexpr int PL = 64 * 64 * (int)sizeof(T) / LINE;             // lines per P block
  static constexpr int SHARED = 3 * WL + PL;
  static constexpr int UL = TW * DmaSlotGeo<T, D>::U_TILE_BYTES / LINE;  // this workgroup's U
  static constexpr int GL = 64 * 4 / LINE;

  // jw: this workgroup's index among the NWG of its (sequence, head); its
  // tiles are TW jw .. TW jw + TW - 1.  touch_shared: the workgroup's share
  // of the lines all NWG workgroups read; touch_own: its U tiles and the
  // gate row.
  __device__ __forceinline__ static void touch_shared(const Args &a, int64_t ch, int h, int jw,
                                                      int lane, unsigned char *junk) {
    const unsigned char *wf = (const unsigned char *)a.Wf + ch * (WL * LINE);
    const unsigned char *kf = (const unsigned char *)a.Kf + k_block(a, ch, h) * (WL * LINE);
    const unsigned char *qf = (const unsigned char *)a.Qf + q_block(a, ch, h) * (WL * LINE);
    const unsigned char *pf = (const unsigned char *)a.Pf + ch * (PL * LINE);
#pragma unroll
    for (int l0 = 0; l0 < SHARED; l0 += NWG * 64) {
      const int l = l0 + jw + NWG * lane;
      const int lc = min(l, SHARED - 1);
      const unsigned char *src = lc < WL ? wf + lc * LINE
                               : lc < 2 * WL ? kf + (lc - WL) * LINE
                               : lc < 3 * WL ? qf + (lc - 2 * WL) * LINE
                               : pf + (lc - 3 * WL) * LINE;
      dma4(src, junk);
    }
  }
  __device__ __forceinline__ static void touch_own(const Args &a, int64_t ch, int jw, int lane,
                                                   unsigned char *junk) {
    const unsigned char *uf = (const unsigned char *)a.Uf + ch * (WL * LINE) +
                              (int64_t)jw * TW * DmaSlotGeo<T, D>::U_TILE_BYTES;
    const unsigned char *gw = (const unsigned char *)(a.Gw + ch * kChunk);
#pragma unroll
    for (int l0 = 0; l0 < UL + GL; l0 += 64) {
      const int l = min(l0 + lane, UL + GL - 1);
      dma4(l < UL ? uf + l * LINE : gw + (l - UL) * LINE, junk);
    }
  }
  __device__ __forceinline__ static void touch(const Args &a, int64_t ch, int h, int jw, int lane,
                                               unsigned char *junk) {
    touch_shared(a, ch, h, jw, lane, junk);
    touch_own(a, ch, jw, lane, junk);
  }
};

// The compute wave's operands when its U tile comes through its own
// registers (four-tile workgroups, whose LDS slots hold W and Ktilde only).
template <typename T, int D, bool SCALE>
struct SlotRegUOps : DmaSlotOps<T, D, 0, SCALE> {
  const T (*u)[4];
  __device__ __forceinline__ f32x4 uvec(int it) const {
    return f32x4{to_f32(u[it][0]), to_f32(u[it][1]), to_f32(u[it][2]), to_f32(u[it][3])};
  }
};

// One chunk's U tile for one lane of a compute wave (result layout, as in
// ChunkOps::load).
template <typename T, int D>
struct UTile {
  T u[4][4];
  __device__ __forceinline__ void load(const Args &a, int64_t ch, int jv, int lane) {
    const T *uf = (const T *)a.Uf + ch * Geo<T, D>::W_ELEMS + (int64_t)jv * 4 * 64 * 4;
#pragma unroll
    for (int it = 0; it < 4; ++it)
      __builtin_memcpy(u[it], uf + ((int64_t)it * 64 + lane) * 4, sizeof(u[it]));
  }
};


// ---------------------------------------------------------------------------
// T form of the four-tile pass (16-bit, D = 128).  With S the chunk-start
// state, K and V the chunk's raw k and v rows, n_t = |k_t| (1 without
// normalisation) and T = (I + A)^-1 from the intra-chunk pass, U = T
// diag(beta) V and W = T diag(beta exp(G)) diag(1/n) K, so
//
//   N            = U - W S = (-T diag(beta)) (diag(exp(G) / n) (K S) - V)
//   Ktilde^T N   = K^T diag(exp(G_last - G) / n) N
//
// and the slot holds the raw k rows (read twice: as rows for K S, and through
// transposed reads for K^T), the workgroup's 64 columns of the raw v rows
// and the 64 x 64 factor -T diag(beta) instead of -W, Ktilde^T and U.  The
// intra-chunk pass then writes 8 KB per chunk-head instead of -W, U (16 KB
// each) and Ktilde^T, and reads no v.  k and v come straight from the input
// (k shared by the sab heads of a k head).  A slot: [k rows][v rows][-T
// diag(beta) fragments][gate row][exp(G)/n row][exp(G_last - G)/n row].  The
// 16-byte units of each k row are permuted by XOR with (row mod 16), those of
// each v row (TW 32-byte tiles, 2 TW units) with (row / (8 / TW) mod 2 TW),
// so every read pattern below (16 rows x 32 bytes at one column offset)
// spreads evenly over the banks.
// ---------------------------------------------------------------------------
template <typename T, int D, int TW>
struct TSlotGeo {
  static_assert(D * (int)sizeof(T) == 256, "sixteen 16-byte units per k row");
  static constexpr int K_BYTES = 64 * 256;
  static constexpr int VROW = TW * 16 * (int)sizeof(T), VU = VROW / 16;   // v row bytes, units
  static constexpr int V_OFF = K_BYTES, V_BYTES = 64 * VROW;
  static constexpr int T_OFF = V_OFF + V_BYTES, T_BYTES = 64 * 64 * (int)sizeof(T);
  static constexpr int G_OFF = T_OFF + T_BYTES;
  static constexpr int R_OFF = G_OFF + 256;       // two rows of 64 floats
  static constexpr int BYTES = R_OFF + 512;
  static constexpr int NK = K_BYTES / 1024, NV = V_BYTES / 1024;
  // the factor's fragments (it, kt) = (0, 1) and (1, 1), rows 0 .. 31 and
  // columns 32 .. 63, lie above the diagonal of a lower-triangular matrix:
  // they are zero, and neither stored nor loaded nor multiplied
  static constexpr int NTF = 6;
  static constexpr int NP = NK + NV + NTF + 3;    // loads per chunk (three 256-byte rows)
  // fragment index (it * 2 + kt) of the j-th loaded factor fragment
  __device__ __forceinline__ static int tfrag(int j) { return j < 2 ? 2 * j : j + 2; }

  // v row r's unit permutation: rows that share banks (256 / VROW of them
  // apart) get different units
  __device__ __forceinline__ static int vswz(int r) { return (r / (256 / VROW)) % VU; }
  // byte offsets in the slot of k row r, elements e .. e + 3, and of v row
  // r, slot columns e .. e + 3 (e % 4 == 0)
  __device__ __forceinline__ static int k_off(int r, int e) {
    return r * 256 + 16 * ((e >> 3) ^ (r & 15)) + 2 * (e & 7);
  }
  __device__ __forceinline__ static int v_off(int r, int e) {
    return V_OFF + r * VROW + 16 * ((e >> 3) ^ vswz(r)) + 2 * (e & 7);
  }
};

// Loader wave `part` of NLD for the T form: piece i of a chunk goes to part
// i % NLD.  k and v rows past the chunk's last token repeat that token's rows
// (their scales and factor columns are zero).
template <typename T, int D, int NLD, int TW>
struct TLoader {
  using SG = TSlotGeo<T, D, TW>;
  static constexpr int PPW = (SG::NP + NLD - 1) / NLD;
  static constexpr int MIN_PER_PART = SG::NP / NLD;
  int lane, part;
  const T *k, *v;    // the sequence's first k row of this k head; v row, first column
  int64_t kstride, vstride;  // elements from one token's row to the next

  __device__ __forceinline__ void issue(const Args &a, int64_t ch, int cc, int len,
                                        unsigned char *slot) const {
    const int rows = min(kChunk, len - kChunk * cc);
    const T *kc = k + (int64_t)kChunk * cc * kstride;
    const T *vc = v + (int64_t)kChunk * cc * vstride;
    const unsigned char *tf = (const unsigned char *)a.Wf + ch * SG::T_BYTES;
#pragma unroll
    for (int m = 0; m < PPW; ++m) {
      const int i = part + NLD * m;
      if (i < SG::NK) {
        // LDS unit p of k row r holds the row's unit p ^ (r % 16)
        const int r = 4 * i + (lane >> 4), p = lane & 15;
        dma16(kc + (int64_t)min(r, rows - 1) * kstride + 8 * (p ^ (r & 15)), slot + i * 1024);
      } else if (i < SG::NK + SG::NV) {
        // LDS unit p of v row r holds the row's unit p ^ vswz(r)
        const int r = (1024 / SG::VROW) * (i - SG::NK) + lane / SG::VU, p = lane % SG::VU;
        dma16(vc + (int64_t)min(r, rows - 1) * vstride + 8 * (p ^ SG::vswz(r)), slot + i * 1024);
      } else if (i < SG::NK + SG::NV + SG::NTF) {
        const int f = SG::tfrag(i - SG::NK - SG::NV);
        dma16(tf + f * 1024 + 16 * lane, slot + SG::T_OFF + f * 1024);
      } else if (i == SG::NK + SG::NV + SG::NTF) {
        dma4(a.Gw + ch * kChunk + lane, slot + SG::G_OFF);
      } else if (i < SG::NP) {
        const int row = i - SG::NK - SG::NV - SG::NTF - 1;
        dma4(a.Bw + ch * 128 + 64 * row + lane, slot + SG::R_OFF + 256 * row);
      }
    }
  }
};

// L2 warm-up of a T-form chunk (one tile per workgroup, intermediates in
// HBM): the NWG workgroups of a (sequence, head) split the 128-byte lines
// every one of them reads -- the chunk's k and v rows (whole rows; rows past
// the chunk's end clamp to its last row, as the loaders do), the factor
// block, the q and P blocks and the three rows -- and touch each once, a
// 4-byte direct load per line into a scratch LDS word, so that the loaders'
// requests a chunk or two later find the lines in L2.
template <typename T, int D, int TW>
struct TWarm {
  static constexpr int NWG = D / 16 / TW;
  static constexpr int LINE = 128, ROWL = D * (int)sizeof(T) / LINE;  // lines per k / v row
  static constexpr int KL = 64 * ROWL, TL = 64 * 64 * (int)sizeof(T) / LINE;
  static constexpr int QL = 64 * D * (int)sizeof(T) / LINE;
  static constexpr int ALL = 2 * KL + TL + QL + TL + 6;  // k, v, factor, q, P, gate and scale rows
  __device__ __forceinline__ static void touch(const Args &a, int64_t ch, int cc, int h, int jw,
                                               int lane, int len, const T *k, const T *v,
                                               int64_t kstride, int64_t vstride,
                                               unsigned char *junk) {
    const int rows = min(kChunk, len - kChunk * cc);
    const unsigned char *kc = (const unsigned char *)(k + (int64_t)kChunk * cc * kstride);
    const unsigned char *vc = (const unsigned char *)(v + (int64_t)kChunk * cc * vstride);
    const unsigned char *tf = (const unsigned char *)a.Wf + ch * (TL * LINE);
    const unsigned char *qf = (const unsigned char *)a.Qf + q_block(a, ch, h) * (QL * LINE);
    const unsigned char *pf = (const unsigned char *)a.Pf + ch * (TL * LINE);
#pragma unroll
    for (int l0 = 0; l0 < ALL; l0 += NWG * 64) {
      const int l = min(l0 + jw + NWG * lane, ALL - 1);
      const unsigned char *src;
      if (l < 2 * KL) {
        const int m = l < KL ? l : l - KL;
        const int r = min(m / ROWL, rows - 1), part = m % ROWL;
        src = l < KL ? kc + (int64_t)r * kstride * (int64_t)sizeof(T) + part * LINE
                     : vc + (int64_t)r * vstride * (int64_t)sizeof(T) + part * LINE;
      } else if (l < 2 * KL + TL) {
        src = tf + (l - 2 * KL) * LINE;
      } else if (l < 2 * KL + TL + QL) {
        src = qf + (l - 2 * KL - TL) * LINE;
      } else if (l < 2 * KL + 2 * TL + QL) {
        src = pf + (l - 2 * KL - TL - QL) * LINE;
      } else {
        const int e = l - 2 * KL - 2 * TL - QL;   // 0, 1: gate row; 2 .. 5: scale rows
        src = e < 2 ? (const unsigned char *)(a.Gw + ch * kChunk) + e * LINE
                    : (const unsigned char *)(a.Bw + ch * 128) + (e - 2) * LINE;
      }
      dma4(src, junk);
    }
  }
};

// One chunk of the recurrence in the T form for compute wave ct's 16-column
// tile (as chunk_step, with the operands of a T-form slot).  The chunk-start
// state and N (unscaled) go to the output waves through xb.
template <typename T, int D, int TW>
__device__ __forceinline__ void tform_step(const unsigned char *slot, int ct,
                                           float (&S)[D / 16][4], int lane,
                                           typename Mfma<T>::frag *xb) {
  using M = Mfma<T>;
  using SG = TSlotGeo<T, D, TW>;
  typedef typename M::frag frag;
  constexpr int KPL = M::KPL, NT = D / 16, KS_D = D / 32, KS_C = 2;
  const int g = lane >> 4, c = lane & 15;
  auto frag2 = [](i16x4 lo, i16x4 hi) {
    return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // With one or two tiles per workgroup (the chain bounds the step) operand
  // reads are issued ahead of the products that use them, so that their
  // latency overlaps earlier products: the k rows of K S up front, the
  // factor's fragments and the row scales during K S, the k columns of K^T
  // during the factor's product (the state does not enter any of them).
  // With four tiles the compiler's own order measured faster (0.198 against
  // 0.203 ms for the GVA batch's state pass).
  constexpr bool early = TW < 4;
  // k rows 16 it + c, dk in pi order (two 8-byte runs): A operands of K S
  frag kr[4][KS_D];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = 16 * it + c, e0 = 32 * kt + 4 * g;
      kr[it][kt] = frag2(*reinterpret_cast<const i16x4 *>(slot + SG::k_off(r, e0)),
                         *reinterpret_cast<const i16x4 *>(slot + SG::k_off(r, e0 + 16)));
    }
  // v rows 16 it + 4 g .. + 3 of this tile's column c (result layout), by
  // transposed reads
  i16x4 v4[4];
#pragma unroll
  for (int it = 0; it < 4; ++it)
    v4[it] = lds_read_tr4(reinterpret_cast<const T *>(slot + SG::v_off(16 * it + 4 * g + (c >> 2),
                                                                         16 * ct + 4 * (c & 3))));
  // the state as operand fragments (dk in pi order), handed to the output waves
  const float *Sflat = &S[0][0];
  frag sb[KS_D];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt) {
    sb[kt] = M::pack(Sflat + kt * KPL);
    xb[kt * 64 + lane] = sb[kt];
  }
  if constexpr (early) __builtin_amdgcn_sched_barrier(0);
  // X = K S, with the factor's fragments read meanwhile
  f32x4 x[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) x[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt)
#pragma unroll
    for (int it = 0; it < 4; ++it) x[it] = M::mma(kr[it][kt], sb[kt], x[it]);
  frag tf[4][KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt)
#pragma unroll
    for (int it = kt > 0 ? 2 : 0; it < 4; ++it)  // (0, 1) and (1, 1) are zero
      tf[it][kt] = *reinterpret_cast<const frag *>(slot + SG::T_OFF +
                                                   ((it * KS_C + kt) * 64 + lane) * 16);
  // rows 16 it + 4 g .. + 3 of exp(G) / n and exp(G_last - G) / n; G_last
  const float *rs = reinterpret_cast<const float *>(slot + SG::R_OFF);
  f32x4 a4[4], b4[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    a4[it] = *reinterpret_cast<const f32x4 *>(rs + 16 * it + 4 * g);
    b4[it] = *reinterpret_cast<const f32x4 *>(rs + 64 + 16 * it + 4 * g);
  }
  const float glast = reinterpret_cast<const float *>(slot + SG::G_OFF)[kChunk - 1];
  if constexpr (early) {
#pragma unroll
    for (int i = 0; i < 7; ++i) {    // 16 products, 15 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two products
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Y = diag(exp(G) / n) X - V (rows 16 it + 4 g + r), as the B operand of
  // the factor's product (t in pi order)
  float yf[16];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const auto vv = __builtin_bit_cast(typename M::half, v4[it]);
#pragma unroll
    for (int r = 0; r < 4; ++r) yf[4 * it + r] = x[it][r] * a4[it][r] - to_f32(vv[r]);
  }
  frag yt[KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt) yt[kt] = M::pack(yf + kt * KPL);
  // N = (-T diag(beta)) Y, with the k columns of K^T (dk rows 16 it + c, t in
  // pi order) read meanwhile through transposed reads
  f32x4 acc[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) acc[it] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt)
#pragma unroll
    for (int it = kt > 0 ? 2 : 0; it < 4; ++it) acc[it] = M::mma(tf[it][kt], yt[kt], acc[it]);
  frag kc[NT][KS_C];
#pragma unroll
  for (int it = 0; it < NT; ++it)
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) {
      const int r0 = 32 * kt + 4 * g + (c >> 2), col = 16 * it + 4 * (c & 3);
      kc[it][kt] = frag2(lds_read_tr4(reinterpret_cast<const T *>(slot + SG::k_off(r0, col))),
                         lds_read_tr4(reinterpret_cast<const T *>(slot + SG::k_off(r0 + 16, col))));
    }
  if constexpr (early) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {    // 6 products, 32 LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);  // five LDS reads
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  float accf[16];
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) accf[4 * it + r] = acc[it][r];
  frag nf[KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt) {
    nf[kt] = M::pack(accf + kt * KPL);
    xb[(KS_D + kt) * 64 + lane] = nf[kt];
  }
  // N's rows scaled by exp(G_last - G_t) / n_t for the update
#pragma unroll
  for (int it = 0; it < 4; ++it)
#pragma unroll
    for (int r = 0; r < 4; ++r) accf[4 * it + r] *= b4[it][r];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt) nf[kt] = M::pack(accf + kt * KPL);
  // S' = exp(G_last) S + K^T (scaled N)
  const float gl = gexp(glast);
#pragma unroll
  for (int it = 0; it < NT; ++it) {
    f32x4 s4 = {S[it][0] * gl, S[it][1] * gl, S[it][2] * gl, S[it][3] * gl};
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) s4 = M::mma(kc[it][kt], nf[kt], s4);
#pragma unroll
    for (int r = 0; r < 4; ++r) S[it][r] = s4[r];
  }
}


// One output wave's operands for one chunk: q fragments of its two token
// tiles, the unmasked P fragments (one for the first tile, two for the
// second) and the gate values of its two rows.
template <typename T, int D>
struct OutRegs {
  typedef typename Mfma<T>::frag frag;
  static constexpr int KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  static constexpr int64_t QBLK = Geo<T, D>::W_ELEMS * sizeof(T) / 16;  // u32x4 per q block
  static constexpr int64_t PBLK = 64 * 64 * sizeof(T) / 16;            // u32x4 per P block
  frag q[2][KS_D];
  frag p0, p1[KS_C];
  float g[2];

  __device__ __forceinline__ void issue(const Args &a, int64_t ch, int h, int lane, int ow) {
    static_assert(KS_C == 2, "64-token chunks: two k-steps over a chunk");
    const int tt0 = ow, tt1 = 3 - ow;
    const frag *qf = reinterpret_cast<const frag *>(reinterpret_cast<const u32x4 *>(a.Qf) +
                                                    q_block(a, ch, h) * QBLK) + lane;
    const frag *pf = reinterpret_cast<const frag *>(reinterpret_cast<const u32x4 *>(a.Pf) + ch * PBLK) + lane;
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt) {
      q[0][kt] = qf[(tt0 * KS_D + kt) * 64];
      q[1][kt] = qf[(tt1 * KS_D + kt) * 64];
    }
    p0 = pf[(tt0 * KS_C) * 64];
#pragma unroll
    for (int kt = 0; kt < KS_C; ++kt) p1[kt] = pf[(tt1 * KS_C + kt) * 64];
    const int c = lane & 15;
    g[0] = a.Gw[ch * kChunk + 16 * tt0 + c];
    g[1] = a.Gw[ch * kChunk + 16 * tt1 + c];
  }
};

// The output values of one chunk for one 16-column tile (output wave ow),
// scaled and rounded, without storing them: res[i] for token tile i.
template <typename T, int D>
__device__ __forceinline__ void output_values(const Args &a, const OutRegs<T, D> &r,
                                              const typename Mfma<T>::frag *xb, int lane, int ow,
                                              typename Mfma<T>::half (&res)[2]) {
  using M = Mfma<T>;
  typedef typename M::frag frag;
  constexpr int KS_D = Geo<T, D>::KS_D, KS_C = Geo<T, D>::KS_C;
  frag sf[KS_D], nf[KS_C];
#pragma unroll
  for (int kt = 0; kt < KS_D; ++kt) sf[kt] = xb[kt * 64 + lane];
#pragma unroll
  for (int kt = 0; kt < KS_C; ++kt) nf[kt] = xb[(KS_D + kt) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < KS_D; ++kt) acc = M::mma(sf[kt], r.q[i][kt], acc);
    const float gam = gexp(r.g[i]);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] *= gam;
    if (i == 0) {
      acc = M::mma(nf[0], r.p0, acc);
    } else {
#pragma unroll
      for (int kt = 0; kt < KS_C; ++kt) acc = M::mma(nf[kt], r.p1[kt], acc);
    }
    f32x4 sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) sc[e] = a.scale * acc[e];
    res[i] = __builtin_convertvector(sc, typename M::half);  // two packed converts
  }
}

// One step of an output wave (st >= 2): fetch chunk st into `into` (past
// the last chunk it repeats the last chunk), then output chunk st - 2 from
// `proc`, fetched two steps earlier, for each of the workgroup's TW column
// tiles (jg0, jg0 + 1, ...).  The step loop below runs whole rounds of the
// three-deep ring without conditions, so the compiler's wait for `proc`
// counts exactly the loads issued after it.
template <typename T, int D, int TW>
__device__ __forceinline__ void output_wave_step(const Args &a, int st, int nc, int len, int sbos,
                                                 int64_t ch0, int jg0, int h, int lane, int ow,
                                                 OutRegs<T, D> &into, const OutRegs<T, D> &proc,
                                                 const typename Mfma<T>::frag (*xbuf)[2][(Geo<T, D>::KS_D + Geo<T, D>::KS_C) * 64]) {
  lds_sync();
  into.issue(a, ch0 + (int64_t)min(st, nc - 1), h, lane, ow);
  const int oc = st - 2;
  const int64_t tok0 = (int64_t)sbos + (int64_t)kChunk * oc;
  const int rows = min(kChunk, len - kChunk * oc);
  if constexpr (TW >= 2) {
    // all tiles' values first, then stores of 16 contiguous bytes per lane:
    // lanes 16 apart (g, g ^ 1) swap halves so that each holds 8 consecutive
    // columns of one tile, and one store writes 64 contiguous bytes of each
    // of 16 rows (two tiles) instead of 32 (GVA batch state pass 0.1995 ->
    // 0.1878 ms; the output stores had cost it 15 %)
    typename Mfma<T>::half res[TW][2];
#pragma unroll
    for (int t = 0; t < TW; ++t) output_values<T, D>(a, proc, xbuf[t][oc & 1], lane, ow, res[t]);
    const int g = lane >> 4, c = lane & 15;
    const bool odd = (g & 1) != 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tt = i == 0 ? ow : 3 - ow;
      const int t = 16 * tt + c;
#pragma unroll
      for (int pr = 0; pr < TW / 2; ++pr) {
        const uint2 lo = __builtin_bit_cast(uint2, res[2 * pr][i]);
        const uint2 hi = __builtin_bit_cast(uint2, res[2 * pr + 1][i]);
        // gfx950's row swap exchanges the odd 16-lane rows of its first
        // operand with the even rows of its second (a VALU op; a shuffle
        // through LDS cost a wait per store): afterwards an even-g lane
        // holds its own tile 2pr columns 4g .. 4g + 3, then the partner's
        // 4g + 4 .. 4g + 7, and an odd-g lane the partner's tile 2pr + 1
        // columns 4g - 4 .. 4g - 1, then its own 4g .. 4g + 3
        const auto sx = __builtin_amdgcn_permlane16_swap(lo.x, hi.x, false, false);
        const auto sy = __builtin_amdgcn_permlane16_swap(lo.y, hi.y, false, false);
        const uint4 v = uint4{sx[0], sy[0], sx[1], sy[1]};
        const int col = 16 * (jg0 + 2 * pr + (odd ? 1 : 0)) + 4 * (g & 2);
        if (t < rows)
          *reinterpret_cast<uint4 *>((T *)a.out + ((tok0 + t) * a.H + h) * D + col) = v;
      }
    }
  } else {
    // one tile: the same row swap pairs the wave's two token tiles instead,
    // so that every lane stores 16 contiguous bytes: an even-g lane columns
    // 4g .. 4g + 7 of its row in token tile ow, an odd-g lane columns
    // 4g - 4 .. 4g + 3 of its row in token tile 3 - ow
    typename Mfma<T>::half res[2];
    output_values<T, D>(a, proc, xbuf[0][oc & 1], lane, ow, res);
    const int g = lane >> 4, c = lane & 15;
    const bool odd = (g & 1) != 0;
    const uint2 lo = __builtin_bit_cast(uint2, res[0]);
    const uint2 hi = __builtin_bit_cast(uint2, res[1]);
    const auto sx = __builtin_amdgcn_permlane16_swap(lo.x, hi.x, false, false);
    const auto sy = __builtin_amdgcn_permlane16_swap(lo.y, hi.y, false, false);
    const uint4 v = uint4{sx[0], sy[0], sx[1], sy[1]};
    const int t = 16 * (odd ? 3 - ow : ow) + c;
    const int col = 16 * jg0 + 4 * (g & 2);
    if (t < rows) *reinterpret_cast<uint4 *>((T *)a.out + ((tok0 + t) * a.H + h) * D + col) = v;
  }
}

constexpr int kFusedLoadWaves = 2;

// Waves of the fused pass: TW = 1 as in the header comment (six waves); TW = 2
// (eight): compute waves 0 and 2 (one per column tile), output waves 1 and 3
// (each for both tiles), loaders 4 and 6, L2 warm-up wave 5, and wave 7 only
// keeps the step barriers.  Waves are dealt to the CU's four SIMDs in turn
// (wave w on SIMD w % 4), so each SIMD holds one matrix-core-heavy wave and
// one light one.  A loader shares the compute wave's SIMD where the loaders,
// not the compute wave, bound the step (the compute wave then waits at the
// step barrier): always with two tiles, and with one tile when the
// intermediates live in HBM (hbm: the L2 warm-up is on), where loader 0
// moves from wave 1 to wave 4 and the warm-up wave to wave 1.
template <int TW> struct FusedRoles;
template <> struct FusedRoles<1> {
  static constexpr int kWaves = 6, kSlots = 4;
  __device__ static int compute_tile(int w) { return w == 0 ? 0 : -1; }
  __device__ static int out_index(int w) { return w == 3 ? 0 : w == 5 ? 1 : -1; }
  __device__ static int warm_wave(bool hbm) { return hbm ? 1 : 4; }
  __device__ static int loader_part(int w, bool hbm) {
    return w == (hbm ? 4 : 1) ? 0 : w == 2 ? 1 : -1;
  }
};
template <> struct FusedRoles<2> {
  static constexpr int kWaves = 8, kSlots = 3;
  __device__ static int compute_tile(int w) { return w == 0 ? 0 : w == 2 ? 1 : -1; }
  __device__ static int out_index(int w) { return w == 1 ? 0 : w == 3 ? 1 : -1; }
  __device__ static int warm_wave(bool) { return 5; }
  __device__ static int loader_part(int w, bool) { return w == 4 ? 0 : w == 6 ? 1 : -1; }
};
// TW = 4 (eight waves): compute waves 0-3 (one per tile and SIMD), output
// waves 4 and 5 (each for all four tiles), loaders 6 and 7.  There is no L2
// warm-up: the GVA batch (8 sequences, 32 heads, 868 MB of intermediates)
// ran 0.480 ms per call without one against 0.524 ms with the output waves
// touching the lines two chunks ahead.
template <> struct FusedRoles<4> {
  static constexpr int kWaves = 8, kSlots = 3;
  __device__ static int compute_tile(int w) { return w < 4 ? w : -1; }
  __device__ static int out_index(int w) { return w == 4 ? 0 : w == 5 ? 1 : -1; }
  __device__ static int warm_wave(bool) { return -1; }
  __device__ static int loader_part(int w, bool) { return w == 6 ? 0 : w == 7 ? 1 : -1; }
};

// TW column tiles per workgroup.  TW = 2 shares the workgroup's W / Ktilde
// loads and its output waves' q / P loads between two tiles, which halves the
// operand traffic per column; it needs a three-slot ring (one chunk ahead
// instead of two) to fit LDS, and is used when the one-tile grid does not fit
// on the CUs at once, so that traffic, not the chain, bounds the pass.
//
// CP: the context-parallel form (k5_cp.hip).  Workgroups cover (sequence,
// segment, head) units instead of (sequence, head); a workgroup runs its
// segment's chunks from the segment's start state in a.cp_start, writes the
// checkpoints that fall inside the segment, and the final state only for the
// segment that holds the sequence's last chunk.  Segments past a sequence's
// end exit at once (segment 0 still runs for an empty sequence, whose final
// state is its initial state).
//
// TF: the T form (no context parallelism; see TSlotGeo).  Its slots hold the
// v rows too, so the compute waves fetch no U.  With one tile per workgroup
// and the intermediates in HBM its warm-up wave touches the chunk's lines two
// chunks ahead (TWarm; 262 144 tokens x 32 heads: state pass 4.64 -> 3.94 ms,
// the same at three chunks ahead, 4.83 ms at one).
template <typename T, int D, int TW, bool CP = false, bool SHK = false, bool TF = false>
__global__ void __launch_bounds__(64 * FusedRoles<TW>::kWaves)
state_output_kernel(Args a) {
  using R = FusedRoles<TW>;
  static_assert(!TF || !CP, "the T form runs without segments");
  constexpr int NT = D / 16, NWG = NT / TW, NLD = kFusedLoadWaves, NSLOT = R::kSlots;
  constexpr int AHEAD = NSLOT - 2;     // chunks the loaders run ahead
  // four tiles: the slots hold W, Ktilde and the gate row, and each compute
  // wave fetches its U tile into registers (LDS holds three such slots and
  // the four tiles' double-buffered hand-off)
  constexpr bool UREG = TW >= 4 && !TF;
  using SGW = DmaSlotGeo<T, D, UREG ? 0 : TW>;
  using LDW = DmaLoader<T, D, NLD, UREG ? 0 : TW>;
  using SLT = std::conditional_t<TF, TSlotGeo<T, D, TW>, SGW>;
  using LDT = std::conditional_t<TF, TLoader<T, D, NLD, TW>, LDW>;
  constexpr int LD_MIN = LDT::MIN_PER_PART;
  typedef typename Mfma<T>::frag frag;
  constexpr int XB = Geo<T, D>::KS_D + Geo<T, D>::KS_C;  // fragments per chunk in xbuf
  static_assert(AHEAD == 1 || AHEAD == 2, "the loader waits below handle one or two chunks ahead");
  static_assert(AHEAD * LD_MIN <= 63, "vmcnt range");
  static_assert(NT % TW == 0, "whole tiles per workgroup");
  __shared__ __align__(16) unsigned char cslots[NSLOT][SLT::BYTES];
  __shared__ frag xbuf[TW][2][XB * 64];
  __shared__ __align__(16) unsigned char junk[256];

  const int b = blockIdx.x;
  const int jw = (b >> 3) % NWG;       // workgroup within its (sequence, head)
  const int jg0 = jw * TW;             // first column tile
  const int H = a.H;
  const int NS = CP ? a.cp_nseg : 1;
  // units in XCD round-robin order (consecutive ids go to the 8 XCDs in turn)
  const int ub = (b / (8 * NWG)) * 8 + (b & 7);
  int u = ub;
  if constexpr (SHK) {
    // the R sab heads of one k head on one XCD, so that the K^T (and q)
    // blocks they share meet in its L2: unit ub = 8 R m + 8 j + x is sab
    // head j of k-head unit 8 m + x (the grid is padded to whole groups)
    const int R = H / a.hk;
    const int ku = (ub / (8 * R)) * 8 + (ub & 7), j = (ub / 8) % R;
    u = (ku / a.hk) * H + (ku % a.hk) * R + j;
    if (ku >= a.N * NS * a.hk) return;
  }
  if (u >= a.N * NS * H) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = u % H;
  const int g = lane >> 4, c = lane & 15;

  int f0, nc, len, sbos;
  const int seq = seq_geometry_by_length(a, u / H / NS, lane, f0, nc, len, sbos);
  // this workgroup's chunks: c0 .. c0 + nc - 1 of the sequence (all of them
  // without CP); len and sbos become the segment's token count and first token
  const int len_seq = len;
  int c0 = 0, seg = 0;
  bool last_seg = true;
  if (CP) {
    seg = (u / H) % NS;
    c0 = seg * a.cp_seg;
    if (seg > 0 && c0 >= nc) return;
    last_seg = c0 + a.cp_seg >= nc;
    nc = min(a.cp_seg, nc - c0);
    len = min(len - kChunk * c0, kChunk * nc);
    sbos += kChunk * c0;
  }
  const int64_t ch0 = ws_index(f0 + c0, h, a.cap);

  const bool hbm = a.warm > 0;
  const int ct = R::compute_tile(wave), ow = R::out_index(wave), part = R::loader_part(wave, hbm);
  if (ct >= 0) {
    // ---------------- compute wave (column tile jg0 + ct) --------------------
    const int jg = jg0 + ct;
    const int vcol = 16 * jg + c;
    int64_t row = seq;
    bool row_ok = true;
    if (a.sidx) {
      row = ld_index(a.sidx, a.sidx_type, seq);
      row_ok = row >= 0 && row < a.pool_rows;
    }
    float S[NT][4];
    if (CP) {
      const int64_t str[4] = {(int64_t)H * D * D, (int64_t)D * D, (int64_t)D, 1};
      read_state_t<float, D>(a.cp_start, str, (int64_t)seq * NS + seg, h, vcol, g, S);
    } else {
      read_state<D>(a, row_ok, row, h, vcol, g, S);
    }
    const int64_t ck_base = a.ck_every > 0 ? ld_index(a.ck_cs, a.ck_cs_type, seq) : 0;
    auto checkpoint = [&](int cc) {
      if (a.ck_every > 0) {
        // tokens of the sequence done after this chunk
        const int done = (c0 + cc + 1) * kChunk;
        if (done <= len_seq && done % a.ck_every == 0) {
          const int64_t crow = ck_base + done / a.ck_every - 1;
          if (crow >= 0 && crow < a.ck_rows)
            write_state<T, D>(a.ck, a.ck_dtype, a.ck_str, crow, h, vcol, g, S);
        }
      }
    };
    if constexpr (UREG) {
      // U tiles in a two-deep register ring: step st works on chunk st - 1
      // and fetches chunk st (the last chunk again at the end); whole rounds
      // of the ring keep the compiler's waits exact
      UTile<T, D> u0, u1;
      auto cstep = [&](int st, const UTile<T, D> &use, UTile<T, D> &fill) {
        fill.load(a, ch0 + (int64_t)min(st, nc - 1), jg, lane);
        lds_sync();
        const int cc = st - 1;
        SlotRegUOps<T, D, SHK> op;
        op.slot = cslots[cc % NSLOT];
        op.lane = lane;
        op.utile = 0;
        op.u = use.u;
        chunk_step<T, D>(a, op, S, ch0 + (int64_t)cc, jg, lane, xbuf[ct][cc & 1]);
        checkpoint(cc);
      };
      if (nc > 0) u0.load(a, ch0, jg, lane);
      lds_sync();
      if (nc > 0) {
        int st = 1;
        for (; st + 2 <= nc + 1; st += 2) {
          cstep(st, u0, u1);
          cstep(st + 1, u1, u0);
        }
        if (st <= nc) cstep(st, u0, u1);
      }
      lds_sync();
    } else {
      for (int st = 0; st <= nc + 1; ++st) {
        lds_sync();
        if (st == 0 || st > nc) continue;
        const int cc = st - 1;
        if constexpr (TF) {
          tform_step<T, D, TW>(cslots[cc % NSLOT], ct, S, lane, xbuf[ct][cc & 1]);
        } else {
          const DmaSlotOps<T, D, TW, SHK> op{cslots[cc % NSLOT], lane, ct};
          chunk_step<T, D>(a, op, S, ch0 + (int64_t)cc, jg, lane, xbuf[ct][cc & 1]);
        }
        checkpoint(cc);
      }
    }
    if (last_seg && a.out_final && a.outst && row_ok)
      write_state<T, D>(a.outst, a.out_dtype, a.out_str, row, h, vcol, g, S);
  } else if (ow >= 0) {
    // ---------------- output waves ------------------------------------------
    OutRegs<T, D> r0, r1, r2;
    if (nc == 0) {
      lds_sync();
      lds_sync();
      return;
    }
    // steps 0 and 1 only fetch; step st >= 2 fetches chunk st and outputs
    // chunk st - 2 (ring slot st % 3 either way)
    lds_sync();
    r0.issue(a, ch0, h, lane, ow);
    lds_sync();
    r1.issue(a, ch0 + (int64_t)min(1, nc - 1), h, lane, ow);
    int st = 2;
    for (; st + 3 <= nc + 2; st += 3) {
      output_wave_step<T, D, TW>(a, st, nc, len, sbos, ch0, jg0, h, lane, ow, r2, r0, xbuf);
      output_wave_step<T, D, TW>(a, st + 1, nc, len, sbos, ch0, jg0, h, lane, ow, r0, r1, xbuf);
      output_wave_step<T, D, TW>(a, st + 2, nc, len, sbos, ch0, jg0, h, lane, ow, r1, r2, xbuf);
    }
    if (st < nc + 2) {
      output_wave_step<T, D, TW>(a, st, nc, len, sbos, ch0, jg0, h, lane, ow, r2, r0, xbuf);
      ++st;
    }
    if (st < nc + 2) output_wave_step<T, D, TW>(a, st, nc, len, sbos, ch0, jg0, h, lane, ow, r0, r1, xbuf);
  } else if ((!TF || TW == 1) && wave == R::warm_wave(hbm)) {
    // ---------------- L2 warm-up wave ---------------------------------------
    const int ahead = a.warm;
    const int kh = h / (H / a.hk), vh = h / (H / a.hv);
    const T *kb = (const T *)a.k + ((int64_t)sbos * a.hk + kh) * D;
    const T *vb = (const T *)a.v + ((int64_t)sbos * a.hv + vh) * D;
    auto touch = [&](int cc) {
      if constexpr (TF)
        TWarm<T, D, TW>::touch(a, ch0 + cc, cc, h, jw, lane, len, kb, vb, (int64_t)a.hk * D,
                               (int64_t)a.hv * D, junk);
      else
        L2Warm<T, D, TW>::touch(a, ch0 + cc, h, jw, lane, junk);
    };
    for (int cc = 0; cc < ahead && cc < nc; ++cc) touch(cc);
    for (int st = 0; st <= nc + 1; ++st) {
      __builtin_amdgcn_s_barrier();
      if (ahead > 0 && st + ahead < nc) touch(st + ahead);
    }
    wait_vm<0>();
  } else if (part >= 0) {
    // ---------------- loader waves ------------------------------------------
    LDT ld;
    if constexpr (TF) {
      const int kh = h / (H / a.hk), vh = h / (H / a.hv);
      ld = LDT{lane, part, (const T *)a.k + ((int64_t)sbos * a.hk + kh) * D,
               (const T *)a.v + ((int64_t)sbos * a.hv + vh) * D + 16 * jg0,
               (int64_t)a.hk * D, (int64_t)a.hv * D};
    } else {
      ld = LDT{(int64_t)jg0 * (SGW::U_TILE_BYTES / 16), lane, part, k_block(a, ch0, h) - ch0};
    }
    auto issue = [&](int cc) {
      if constexpr (TF) ld.issue(a, ch0 + (int64_t)cc, cc, len, cslots[cc % NSLOT]);
      else ld.issue(a, ch0 + (int64_t)cc, cslots[cc % NSLOT]);
    };
    for (int cc = 0; cc < AHEAD && cc < nc; ++cc) issue(cc);
    for (int st = 0; st <= nc + 1; ++st) {
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      if (st + AHEAD < nc) issue(st + AHEAD);
      // chunk st must have landed before the next barrier; the loads issued
      // after it (up to AHEAD newer chunks where they exist) may stay in flight
      if (st < nc) {
        const int newer = min(AHEAD, nc - 1 - st);
        if (newer >= 2) wait_vm<2 * LD_MIN>();
        else if (newer == 1) wait_vm<LD_MIN>();
        else wait_vm<0>();
      }
    }
  } else {
    // ---------------- barrier-only wave -------------------------------------
    for (int st = 0; st <= nc + 1; ++st) __builtin_amdgcn_s_barrier();
  }
}

template <typename T, int D, int TW, bool TF = false>
static hipError_t launch_state_output_tw(const Args &a, hipStream_t s) {
  constexpr int NWG = D / 16 / TW;
  const bool cp = a.cp_nseg > 0;
  const int64_t ns = cp ? a.cp_nseg : 1;
  const int64_t units = (int64_t)a.N * a.H * ns;
  int64_t blocks = ((units + 7) / 8) * 8 * NWG;
  if (a.H != a.hk) {
    // k-head groups of H / hk units, whole groups of 8 (see the kernel)
    const int64_t kunits = (int64_t)a.N * a.hk * ns;
    blocks = ((kunits + 7) / 8) * 8 * (a.H / a.hk) * NWG;
  }
  const dim3 grid((unsigned)blocks), block(64 * FusedRoles<TW>::kWaves);
  const bool shk = a.H != a.hk;   // sab heads share k heads (GQA / GVA)
  if constexpr (TF) {
    if (cp) return hipErrorInvalidValue;
    if (shk) state_output_kernel<T, D, TW, false, true, true><<<grid, block, 0, s>>>(a);
    else state_output_kernel<T, D, TW, false, false, true><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
  }
  if constexpr (D == 128) {
    if (cp) {
      if (shk) state_output_kernel<T, D, TW, true, true><<<grid, block, 0, s>>>(a);
      else state_output_kernel<T, D, TW, true, false><<<grid, block, 0, s>>>(a);
      return hipGetLastError();
    }
  } else {
    if (cp) return hipErrorInvalidValue;
  }
  if (shk) state_output_kernel<T, D, TW, false, true><<<grid, block, 0, s>>>(a);
  else state_output_kernel<T, D, TW, false, false><<<grid, block, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_state_output_t(const Args &a, hipStream_t s) {
  constexpr int NT = D / 16;
  const int64_t units = (int64_t)a.N * a.H * (a.cp_nseg > 0 ? a.cp_nseg : 1);
  if (units == 0) return hipSuccess;
  // one workgroup per CU (LDS): two tiles per workgroup once the one-tile
  // grid no longer fits on the CUs at once (the GVA batch with 32 heads and 8
  // sequences: 0.427 -> 0.317 ms); up to that the chain bounds the pass and
  // one tile per workgroup spreads it over more CUs.  Four tiles once even
  // the four-tile grid covers every CU: the operand traffic per column halves
  // again.
  const int64_t cus = a.num_cus > 0 ? a.num_cus : 1;
  const int tw = (NT % 4 == 0 && units * NT >= 4 * cus) ? 4 : units * NT > cus ? 2 : 1;
  // the T form (chosen by the host with the intra-chunk pass's output form)
  if constexpr (D == 128) {
    if (a.tform) {
      if (tw == 4) return launch_state_output_tw<T, D, 4, true>(a, s);
      if (tw == 2) return launch_state_output_tw<T, D, 2, true>(a, s);
      return launch_state_output_tw<T, D, 1, true>(a, s);
    }
  } else {
    if (a.tform) return hipErrorInvalidValue;
  }
  if constexpr (NT % 4 == 0) {
    if (tw == 4) return launch_state_output_tw<T, D, 4>(a, s);
  }
  if (tw == 2) return launch_state_output_tw<T, D, 2>(a, s);
  return launch_state_output_tw<T, D, 1>(a, s);
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
