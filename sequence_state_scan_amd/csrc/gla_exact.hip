// Exact sub-block kernels: the chunk form for any log-gate g <= 0.
//
// The fast kernels factor exp(b_t - b_s) inside a chunk as exp(b_t) * exp(-b_s) (the K/Lambda
// form the ZeCO referee report compares with K*Gamma in its minor comment 4).  That needs
// exp(-b) to stay finite, so a chunk in which a channel decays by more than a fixed bound is
// handed to the kernels here, which never form a growing exponential:
//   - every chunk is walked in sub-blocks of 16 tokens; b is the inclusive running sum of g inside
//     the sub-block and lam its total;
//   - across sub-blocks the state carries the history: O = Qbar S + A V with Qbar = q exp(b), and
//     S <- exp(lam) S + Ktil^T V with Ktil = k exp(lam - b) (all factors <= 1);
//   - inside a sub-block the scores are summed element by element,
//       A[t][s] = sum_c q_tc k_sc exp(b_tc - b_sc)   (s <= t, exponent <= 0),
//     by the 16 lanes of a row (one token each) broadcasting k_s and b_s along the row with DPP.
// The backward walks the same sub-blocks in reverse.  It needs the state before every sub-block:
// it reloads the stored global state before the chunk and advances it through the chunk's earlier
// sub-blocks (no division by a decay is ever needed).  Per sub-block, with U = dL/dS after it:
//   dq = exp(b) (S do) + sum_{s <= t} dA[t][s] k_s exp(b_t - b_s)
//   dk = exp(lam - b) (U v) + sum_{t >= s} dA[t][s] q_t exp(b_t - b_s)
//   dv = A^T dO + Ktil U
//   U <- exp(lam) U + Qbar^T dO
//   dg_t = sum_{t' >= t in the sub-block} (q dq - k dk)_t' + rowsum(S_after * U_after)
// (the last line is the exact carry of the fast backward, at sub-block granularity, formed the
// same way: rowsum(S_before * exp(lam) U) + sum_s (k dk|U)_s).
//
// One workgroup of 8 waves per unit (b, h, segment); with flags non-null only the units whose
// flag is 1 (set by the fast kernel) run.  With a re-split list, further workgroups serve the
// pieces of the listed flagged units, each from its true incoming state (unit_place).  These
// kernels favour simplicity over speed: they serve chunks of 16 tokens in bf16, and units with
// strongly decaying channels.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

namespace {

constexpr int kMaxChunk = 64;
constexpr int kSB = 16;  // tokens per sub-block
constexpr float kLog2e = 1.44269504088896341f;

// exp(b_t - b_s) or exp(b_s - b_t), whichever exponent is not positive, from b in base 2 (b2 = b log2 e):
// b does not rise along a sub-block (the gates are <= 0), so this is exp(b_t - b_s) for s <= t and
// exp(b_s - b_t) for s >= t, up to the rounding of the prefix sums.  One v_exp_f32 with a -|x|
// operand modifier.
__device__ __forceinline__ float exp_nonpos(float b2t, float b2s) { return __builtin_amdgcn_exp2f(-fabsf(b2t - b2s)); }

// b in base 2.  The values are hidden from the optimiser, so that b2_t - b2_s stays one subtraction
// (with the broadcast of b2_s folded into it) rather than a multiply-add that recomputes b2_t.
__device__ __forceinline__ f32x4 base2(f32x4 b) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v = b[e] * kLog2e;
    asm volatile("" : "+v"(v));
    r[e] = v;
  }
  return r;
}

// Gate item of a 16-token sub-block: thread (row R = tid / 16, lane t = tid % 16) holds token t's
// q, k and g for the channels 4R .. 4R + 3; rows R < DK / 4 take part (others hold zeros).
template <typename E>
struct SubGate {
  f32x4 q, k, b, lam;  // b: inclusive running sum of g inside the sub-block; lam: its total
  // the loads alone (b holds the raw gate until scan())
  __device__ __forceinline__ void fetch(const E* qp, const E* kp, const float* gp, long tok, int DK, int R,
                                        bool act) {
    b = q = k = zero4();
    if (act) {
      const long off = tok * DK + 4 * R;
      q = load4(qp + off);
      k = load4(kp + off);
      b = load4(gp + off);
    }
  }
  __device__ __forceinline__ void scan() {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      b[e] = seg_scan_incl<16>(b[e]);
      lam[e] = seg_last<16>(b[e]);
    }
  }
  __device__ __forceinline__ void load(const E* qp, const E* kp, const float* gp, long tok, int DK, int R,
                                       bool act) {
    fetch(qp, kp, gp, tok, DK, R, act);
    scan();
  }
};

// part[s] = sum over the thread's 4 channels of q_t k_s exp(b_t - b_s) for s <= t, 0 for s > t.
template <typename E>
__device__ __forceinline__ void diag_parts(const SubGate<E>& x, int t, float (&part)[16]) {
  const f32x4 b2 = base2(x.b);
  static_for<0, 16>([&](auto S) {
    constexpr int s = decltype(S)::value;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += x.q[e] * (row_bcast<s>(x.k[e]) * exp_nonpos(b2[e], row_bcast<s>(b2[e])));
    part[s] = s <= t ? acc : 0.f;  // the s > t terms are dropped
    __builtin_amdgcn_sched_barrier(0);  // one s at a time: bounded register use
  });
}

// The parts summed over the 4 lane rows of the wave (reduce-scatter): lane row g4 ends with the
// sums of s = 4 g4 .. 4 g4 + 3 in r[0..3].
__device__ __forceinline__ f32x4 reduce_scores(const float (&part)[16]) {
  const int g4 = lane_id() >> 4, hi = g4 >> 1, lo = g4 & 1;
  float r1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float mine = hi ? part[8 + i] : part[i], other = hi ? part[i] : part[8 + i];
    r1[i] = mine + __shfl_xor(other, 32);
  }
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float mine = lo ? r1[4 + i] : r1[i], other = lo ? r1[i] : r1[4 + i];
    r[i] = mine + __shfl_xor(other, 16);
  }
  return r;
}

// A sub-block's gate items, and one 8-element piece per thread of a [token][DV] tensor of the
// sub-block (V in the forward, dO in the backward; threads beyond the NP pieces re-read the last
// one, which they never store), issued ahead of their use.
template <typename E, int DK, int DV, int NP>
__device__ __forceinline__ void fetch_sub_block(SubGate<E>& x, Vec8<E>& piece, const E* q, const E* k, const float* g,
                                                const E* rows, long ts, int tid, bool act) {
  x.fetch(q, k, g, ts + (tid & 15), DK, tid >> 4, act);
  const int pc = tid < NP ? tid : NP - 1;
  piece.load(rows + (ts + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
}

// The lane's 4 accumulator columns of a state tile pair / piece from the tiled chunk-state layout
// (U's lane layout: row 16 cb + n16, columns 16 jb + 4 g4 .. + 3), widened to float.
template <typename E, int NJB>
__device__ __forceinline__ void load_state_rows(const E* st, int cb, f32x4 (&S)[NJB]) {
  const int l = lane_id(), L = state_lane_row(l & 15, l >> 4);
  if constexpr (NJB % 2 == 0) {
#pragma unroll
    for (int m = 0; m < NJB / 2; ++m) {
      typename Piece4<E>::type x, y;
      load_state_pair<E, NJB>(st, cb, m, L, x, y);
      S[2 * m] = widen(x);
      S[2 * m + 1] = widen(y);
    }
  } else {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) S[jb] = widen(load_state_piece<E, NJB>(st, cb, jb, L));
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------
// Forward: local pass of every segment from a zero state (same results as fwd_local_kernel).
// Wave w owns the JPW column blocks JPW w .. of the float32 state (all rows), as in the fast kernel.
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_exact_kernel(FwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  constexpr int NJB = DV / 16, NKB = DK / 16, JPW = ceil_div(NJB, NW);
  constexpr int NGR = DK / 4, NGW = ceil_div(NGR, 4);  // gate rows, waves holding them
  constexpr int LDQ = lds_ld<E>(DK), LDV = lds_ld<E>(DV), LDA = lds_ld<E>(kSB);
  constexpr int NVP = kSB * DV / 8, VPT = ceil_div(NVP, NT);
  static_assert(JPW == 1 || NJB % NW == 0, "a wave owns JPW column blocks, or none");
  static_assert(NGR <= NT / 16, "one gate row per 4 channels");

  __shared__ __attribute__((aligned(16))) E sQb[kSB * LDQ];  // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sQh[kSB * LDQ];  // q exp(b - lam) [t][c] (scores on MFMA)
  __shared__ __attribute__((aligned(16))) E sKt[kSB * LDQ];  // Ktil [s][c]
  __shared__ __attribute__((aligned(16))) E sV[kSB * LDV];   // V [s][j]
  __shared__ __attribute__((aligned(16))) E sA[kSB * LDA];   // A [t][s], masked
  __shared__ __attribute__((aligned(16))) float sRed[NGW][kSB][kSB];  // per-wave partial scores
  __shared__ __attribute__((aligned(16))) float sLamE[DK];            // exp(lam)
  __shared__ __attribute__((aligned(8))) unsigned char sMod[8];       // per wave: see post_moderate
  static_assert(NW <= 8, "one verdict byte per wave");

  const UnitPlace up = unit_place(a, n_units, DK, (long)DK * DV);
  if (!up.live) return;
  if (!up.X && a.flags && a.flags[up.unit] == 0) return;  // the fast kernel has done this unit
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  E* __restrict__ o = static_cast<E*>(a.o);
  E* __restrict__ cst = static_cast<E*>(a.chunk_states);
  const int C = a.chunk, NSB = C / kSB;
  const int unit = up.unit, NS = up.NS, sub = up.sub, seg = up.seg;  // sub-segments, as in fwd_local_kernel
  const int L = a.T / a.P, Ls = L / NS, nchunks = Ls / C;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L + (long)sub * Ls;
  const long chunk0 = tok0 / C;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const int R = tid >> 4, t = n16;
  const bool gact = R < NGR, vrole = w * JPW < NJB;

  f32x4 S[JPW][NKB];  // S[jj][kb][i] = S[16kb + 4g4 + i][16jb + n16], jb = JPW w + jj
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      if (up.init && (sub > 0 || a.from_in) && vrole)  // the state entering the sub-segment
        S[jj][kb] = quad_transpose(load4(up.init + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV +
                                         (w * JPW + jj) * 16 + (n16 & ~3)));
      else
        S[jj][kb] = zero4();
    }
  f32x4 ldsum = zero4();  // log cumulative decay of the segment, channels 4R ..

  // the next sub-block's gate items and V piece, fetched one sub-block ahead of their use (the walk
  // goes forwards through contiguous chunks: the next sub-block is always the next 16 tokens)
  static_assert(VPT == 1, "one piece of a sub-block's V per thread");
  SubGate<E> xn;
  Vec8<E> pvn;
  fetch_sub_block<E, DK, DV, NVP>(xn, pvn, q, k, a.g, v, tok0, tid, gact);
  // Whether every channel of the sub-block whose raw gates xr holds decays by at most
  // exp(kFastMinChunkLogDecay): sufficient is that none of its 16 log-gates is below a 16th of that.
  // Each wave posts its verdict in sMod for the next sub-block before the barrier that ends the
  // current one, so the choice between the two forms of the scores needs no barrier of its own.
  constexpr float kModerateGate = kFastMinChunkLogDecay / kSB;
  constexpr unsigned long long kAllModerate = (NW == 8 ? ~0ull : (1ull << (8 * NW)) - 1) & 0x0101010101010101ull;
  auto post_moderate = [&](const SubGate<E>& xr) {
    const bool ok = xr.b[0] >= kModerateGate && xr.b[1] >= kModerateGate && xr.b[2] >= kModerateGate &&
                    xr.b[3] >= kModerateGate;
    const bool wave_ok = __ballot(!ok) == 0;
    if (lane_id() == 0) sMod[w] = wave_ok ? 1 : 0;
  };
  post_moderate(xn);
  __syncthreads();

  for (int n = 0; n < nchunks; ++n) {
    for (int j = 0; j < NSB; ++j) {
      const long ts0 = tok0 + (long)n * C + j * kSB;
      const bool moderate = (*reinterpret_cast<const unsigned long long*>(sMod) & kAllModerate) == kAllModerate;
      // ---- gate prefix, Qbar, Ktil, V -> LDS; the scores of the sub-block ----
      SubGate<E> x = xn;
      x.scan();
      if (NVP == NT || tid < NVP) pvn.store(sV + (tid / (DV / 8)) * LDV + (tid % (DV / 8)) * 8);
      const bool more = n < nchunks - 1 || j < NSB - 1;
      if (more) fetch_sub_block<E, DK, DV, NVP>(xn, pvn, q, k, a.g, v, ts0 + kSB, tid, gact);
      if (gact) {
        f32x4 xq, xk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[e] = x.q[e] * __expf(x.b[e]);
          xk[e] = x.k[e] * __expf(x.lam[e] - x.b[e]);
        }
        store4(sQb + t * LDQ + 4 * R, xq);
        store4(sKt + t * LDQ + 4 * R, xk);
        if (moderate) {
          f32x4 xh;
#pragma unroll
          for (int e = 0; e < 4; ++e) xh[e] = x.q[e] * __expf(x.b[e] - x.lam[e]);
          store4(sQh + t * LDQ + 4 * R, xh);
        }
        if (t == 0) {
          f32x4 le;
#pragma unroll
          for (int e = 0; e < 4; ++e) le[e] = __expf(x.lam[e]);
          store4(sLamE + 4 * R, le);
        }
        ldsum += x.lam;
      }
      if (moderate) {
        // A = (q exp(b - lam)) (k exp(lam - b))^T on one MFMA tile, as the fast kernels factor it
        // (both factors within exp(40) here), masked to s <= t
        __syncthreads();
        if (w == 0) {
          const f32x4 acc = mma<E, false, false>(zero4(), sQh, LDQ, sKt, LDQ, 0, DK);
#pragma unroll
          for (int i = 0; i < 4; ++i) sA[(4 * g4 + i) * LDA + n16] = (E)(n16 <= 4 * g4 + i ? acc[i] : 0.f);
        }
      } else {
        // element by element, every exponent non-positive
        if (w < NGW) {
          float part[16];
          diag_parts(x, t, part);
          const f32x4 r = reduce_scores(part);
          *reinterpret_cast<f32x4*>(&sRed[w][t][4 * g4]) = r;
        }
        __syncthreads();
        if (tid < kSB * kSB) {
          const int tt = tid >> 4, ss = tid & 15;
          float acc = 0.f;
#pragma unroll
          for (int ww = 0; ww < NGW; ++ww) acc += sRed[ww][tt][ss];
          sA[tt * LDA + ss] = (E)acc;
        }
      }
      __syncthreads();
      // ---- O^T[j][t] = V^T A^T + S^T Qbar^T; S = diag(exp(lam)) S + Ktil^T V ----
      if (vrole) {
        f32x4 acc[JPW];
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj)
          acc[jj] = mma_k16<E, true, false>(zero4(), sV + (w * JPW + jj) * 16, LDV, sA, LDA);
        if constexpr (sizeof(E) == 2) {
#pragma unroll
          for (int pp = 0; pp < NKB / 2; ++pp) {
            const bf16x8 y = *reinterpret_cast<const bf16x8*>(sQb + n16 * LDQ + 32 * pp + pair_col(g4));
#pragma unroll
            for (int jj = 0; jj < JPW; ++jj)
              acc[jj] = Mma<bf16>::mma(merge_pair(to_bf16x4(S[jj][2 * pp]), to_bf16x4(S[jj][2 * pp + 1])), y, acc[jj]);
          }
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) {
            f32x4 one[1] = {acc[jj]};
            mma_regX_rows<NKB, 1>(one, S[jj], sQb + n16 * LDQ, 16 * LDQ);
            acc[jj] = one[0];
          }
        }
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) store4(o + (ts0 + n16) * DV + (w * JPW + jj) * 16 + 4 * g4, acc[jj]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const f32x4 le = load4(sLamE + kb * 16 + 4 * g4);
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            S[jj][kb] = mma_k16<E, true, true>(S[jj][kb] * le, sKt + kb * 16, LDQ, sV + (w * JPW + jj) * 16, LDV);
        }
      }
      if (more) post_moderate(xn);  // every wave has read sMod for this sub-block before its first barrier
      __syncthreads();
    }
    // ---- the local state after the chunk, in the tiled chunk-state layout (none kept for a
    // forward-only caller) ----
    if (vrole && cst) {
      E* cs = cst + (chunk0 + n) * (long)DK * DV;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (JPW == 2) {
          store_state_pair<E, NJB>(cs, kb, w, state_lane_qt(n16, g4), quad_transpose(S[0][kb]),
                                   quad_transpose(S[1][kb]));
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            store_state_piece<E, NJB>(cs, kb, w * JPW + jj, state_lane_qt(n16, g4), quad_transpose(S[jj][kb]));
        }
      }
    }
  }
  // ---- segment results: local end state (float32) and log cumulative decay (with from_in the
  // state pass has given them) ----
  if (a.from_in) {
  } else if (NS == 1) {
    if (vrole) {
      float* st = a.seg_state + (long)unit * DK * DV;
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          store4(st + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + (w * JPW + jj) * 16 + (n16 & ~3),
                 quad_transpose(S[jj][kb]));
    }
    if (gact && t == 0) store4(a.seg_logdecay + (long)unit * DK + 4 * R, ldsum);
  } else if (sub == NS - 1) {
    // the end state comes from the scan over the sub-segments; the log decay is their sum
    for (int c = tid; c < DK; c += NW * 64) {
      float sum = 0.f;
      for (int s2 = 0; s2 < up.nld; ++s2) sum += up.ldb[(long)s2 * DK + c];
      a.seg_logdecay[(long)seg * DK + c] = sum;
    }
  }
}

// ------------------------------------------------------------------------------------------------
// Backward of every segment given the global chunk states (same results as bwd_kernel).
// Wave w < DK/16 holds rows c = 16w .. of U (all of d_v) and of the state before the sub-block, in
// the lane layout U[16w + n16][16jb + 4g4 + i]; its 4 gate rows hold the channels 16w + 4g4 + i of
// token n16, which is exactly the accumulator layout of the dq and dk products.
// ------------------------------------------------------------------------------------------------
template <typename E, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_exact_kernel(BwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  constexpr int NJB = DV / 16, NCB = DK / 16;
  constexpr int LDQ = lds_ld<E>(DK), LDV = lds_ld<E>(DV), LDA = lds_ld<E>(kSB), LDU = lds_ld<E>(DV);
  constexpr int NVC = kMaxChunk * DV / 8, NVS = kSB * DV / 8;  // 8-element pieces of V (chunk), dO (sub-block)
  static_assert(NCB <= NW, "one 16-row block of U per wave");
  static_assert(sizeof(E) == 4 || NJB % 2 == 0, "d_v blocks pair up for bf16");

  constexpr int SZ_U = DK * LDU * (int)sizeof(E), SZ_RED = NCB * kSB * kSB * 4;
  __shared__ __attribute__((aligned(16))) E sKt[kMaxChunk * LDQ];  // Ktil [s][c], whole chunk
  __shared__ __attribute__((aligned(16))) E sQb[kMaxChunk * LDQ];  // Qbar [t][c], whole chunk
  __shared__ __attribute__((aligned(16))) E sV[kMaxChunk * LDV];   // V [s][j], whole chunk
  __shared__ __attribute__((aligned(16))) E sdO[kSB * LDV];        // dO [t][j], sub-block
  __shared__ __attribute__((aligned(16))) E sA[kSB * LDA];         // A [t][s], masked
  __shared__ float sdA[kSB][kSB + 1];                               // dA [t][s], masked
  __shared__ __attribute__((aligned(16))) E sQh[kSB * LDQ];        // q exp(b - lam) [t][c], sub-block
  __shared__ __attribute__((aligned(16))) E sdAb[kSB * LDA];       // dA [t][s], masked, element type
  __shared__ __attribute__((aligned(8))) unsigned char sMod[8];     // per wave: see post_moderate
  static_assert(NW <= 8, "one verdict byte per wave");
  __shared__ __attribute__((aligned(16))) float sLamE[kMaxChunk / kSB][DK];  // exp(lam) per sub-block
  __shared__ __attribute__((aligned(16))) unsigned char sUR[SZ_U > SZ_RED ? SZ_U : SZ_RED];
  E* const sU = reinterpret_cast<E*>(sUR);                            // U [c][j], after the scores
  float (*const sRed)[kSB][kSB] = reinterpret_cast<float (*)[kSB][kSB]>(sUR);  // per-wave partial scores

  const UnitPlace up = unit_place(a, n_units, DK, (long)DK * DV);
  if (!up.live) return;
  if (!up.X && a.flags && a.flags[up.unit] == 0) return;  // the fast kernel has done this unit
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const E* __restrict__ dO = static_cast<const E*>(a.dO);
  const E* __restrict__ cst = static_cast<const E*>(a.chunk_states);
  E* __restrict__ dq = static_cast<E*>(a.dq);
  E* __restrict__ dk = static_cast<E*>(a.dk);
  E* __restrict__ dv = static_cast<E*>(a.dv);
  const int C = a.chunk, NSB = C / kSB;
  const int unit = up.unit, NS = up.NS, sub = up.sub, seg = up.seg;  // sub-segments, as in bwd_kernel
  const int L = a.T / a.P, Ls = L / NS, nchunks = Ls / C;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L + (long)sub * Ls;
  const long chunk0 = tok0 / C;
  constexpr long SS = (long)DK * DV;
  const int w = wave_id();
  const bool urole = w < NCB;  // holds U rows 16w .. and the gate rows 4w .. 4w + 3

  f32x4 U[NJB];  // U[jb][i] = U[16w + n16][16jb + 4g4 + i]
  if (up.init && (sub < NS - 1 || a.from_in) && urole) {
    // the gradient w.r.t. the state leaving the sub-segment (from the rest of its segment, or the
    // global one with from_in)
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) U[jb] = load4(up.init + (long)(16 * w + n16) * DV + jb * 16 + 4 * g4);
  } else {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) U[jb] = zero4();
  }

  // the next sub-block's gate items and dO piece, fetched one sub-block ahead of their use; the walk
  // goes backwards through contiguous chunks, so the next sub-block is always the previous 16 tokens
  static_assert(NVS <= NT, "one piece of a sub-block's dO per thread");
  SubGate<E> xn;
  Vec8<E> pdn;
  fetch_sub_block<E, DK, DV, NVS>(xn, pdn, q, k, a.g, dO, tok0 + (long)(nchunks - 1) * C + (NSB - 1) * kSB, threadIdx.x,
                                   urole);
  // Whether every channel of the sub-block whose raw gates xr holds decays by at most
  // exp(kFastMinChunkLogDecay), as in the forward: posted per wave for the next sub-block before the
  // barrier that ends the current one
  constexpr float kModerateGate = kFastMinChunkLogDecay / kSB;
  constexpr unsigned long long kAllModerate = (NW == 8 ? ~0ull : (1ull << (8 * NW)) - 1) & 0x0101010101010101ull;
  auto post_moderate = [&](const SubGate<E>& xr) {
    const bool ok = xr.b[0] >= kModerateGate && xr.b[1] >= kModerateGate && xr.b[2] >= kModerateGate &&
                    xr.b[3] >= kModerateGate;
    const bool wave_ok = __ballot(!ok) == 0;
    if (lane_id() == 0) sMod[w] = wave_ok ? 1 : 0;
  };
  post_moderate(xn);
  __syncthreads();

  for (int n = nchunks - 1; n >= 0; --n) {
    const long tc0 = tok0 + (long)n * C;
    const int tid = fresh_tid(), R = tid >> 4, t = tid & 15;
    // ---- the chunk's Qbar, Ktil, exp(lam) per sub-block, and V -> LDS ----
    for (int j = 0; j < NSB; ++j) {
      SubGate<E> x;
      x.load(q, k, a.g, tc0 + j * kSB + t, DK, R, urole);
      if (urole) {
        f32x4 xq, xk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xq[e] = x.q[e] * __expf(x.b[e]);
          xk[e] = x.k[e] * __expf(x.lam[e] - x.b[e]);
        }
        store4(sQb + (j * kSB + t) * LDQ + 4 * R, xq);
        store4(sKt + (j * kSB + t) * LDQ + 4 * R, xk);
        if (t == 0) {
          f32x4 le;
#pragma unroll
          for (int e = 0; e < 4; ++e) le[e] = __expf(x.lam[e]);
          store4(&sLamE[j][4 * R], le);
        }
      }
    }
    for (int pc = tid; pc < NVC; pc += NT) {
      if (pc / (DV / 8) >= C) break;
      Vec8<E> pv;
      pv.load(v + (tc0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
      pv.store(sV + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
    }
    __syncthreads();
    for (int j = NSB - 1; j >= 0; --j) {
      const long ts0 = tc0 + j * kSB;
      // lane indices re-derived here, so the per-lane addresses are not held across the loop
      const int tid = fresh_tid(), l = tid & 63, n16 = l & 15, g4 = l >> 4, R = tid >> 4, t = n16;
      const bool moderate = (*reinterpret_cast<const unsigned long long*>(sMod) & kAllModerate) == kAllModerate;
      SubGate<E> x = xn;  // fetched one sub-block ahead
      x.scan();
      if (NVS == NT || tid < NVS) pdn.store(sdO + (tid / (DV / 8)) * LDV + (tid % (DV / 8)) * 8);
      const bool more = n > 0 || j > 0;
      if (more) fetch_sub_block<E, DK, DV, NVS>(xn, pdn, q, k, a.g, dO, ts0 - kSB, tid, urole);
      if (moderate && urole) {
        f32x4 xh;
#pragma unroll
        for (int e = 0; e < 4; ++e) xh[e] = x.q[e] * __expf(x.b[e] - x.lam[e]);
        store4(sQh + t * LDQ + 4 * R, xh);
      }
      __syncthreads();
      // the stored global state before the chunk, requested here and used after the element-wise
      // sums (the segment's first chunk starts from seg_in, read where it is used)
      const bool from_store = n > 0 || sub > 0;
      typename Piece4<E>::type Sc[NJB];
      if (urole && from_store) {
        const E* st = cst + (chunk0 + n - 1) * SS;
        const int L = state_lane_row(n16, g4);
        if constexpr (NJB % 2 == 0) {
#pragma unroll
          for (int m = 0; m < NJB / 2; ++m) load_state_pair<E, NJB>(st, w, m, L, Sc[2 * m], Sc[2 * m + 1]);
        } else {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) Sc[jb] = load_state_piece<E, NJB>(st, w, jb, L);
        }
      }
      // ---- dA[t][s] = dO_t . V_s (s <= t) ----
      if (w == 0) {
        const f32x4 acc = mma<E, false, false>(zero4(), sdO, LDV, sV + j * kSB * LDV, LDV, 0, DV);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d = n16 <= 4 * g4 + i ? acc[i] : 0.f;
          sdA[4 * g4 + i][n16] = d;
          if (moderate) sdAb[(4 * g4 + i) * LDA + n16] = (E)d;
        }
      }
      __syncthreads();
      f32x4 dqd = zero4(), dkd = zero4();
      if (moderate) {
        // ---- a sub-block that decays by at most exp(-40): the fast kernels' factoring on MFMA tiles.
        // Scores A = (q exp(b - lam)) Ktil^T; dq's intra part exp(b_t - lam) (dA Ktil)[t]; dk's
        // exp(-b_s) (dA^T Qbar)[s] (every factor within exp(40)) ----
        if (w == 0) {
          const f32x4 acc = mma<E, false, false>(zero4(), sQh, LDQ, sKt + j * kSB * LDQ, LDQ, 0, DK);
#pragma unroll
          for (int i = 0; i < 4; ++i) sA[(4 * g4 + i) * LDA + n16] = (E)(n16 <= 4 * g4 + i ? acc[i] : 0.f);
        }
        if (urole) {
          const f32x4 aq = mma_k16<E, true, false>(zero4(), sKt + j * kSB * LDQ + 16 * w, LDQ, sdAb, LDA);
          const f32x4 ak = mma_k16<E, true, true>(zero4(), sQb + j * kSB * LDQ + 16 * w, LDQ, sdAb, LDA);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            dqd[i] = __expf(x.b[i] - x.lam[i]) * aq[i];
            dkd[i] = __expf(-x.b[i]) * ak[i];
          }
        }
      } else if (urole) {
        // ---- element-wise sums inside the sub-block: scores, and the intra parts of dq and dk ----
        // one exponential per (t, s, channel) serves the scores, dq and dk: exp(b_t - b_s) for s <= t
        // (scores and dq), exp(b_s - b_t) for s >= t (dk).  dA is masked (zero for s > t), so
        // dA[t][s] keeps dq to s <= t and dA[s][t] keeps dk to s >= t; the scores' s > t terms are
        // dropped by the select below.
        const f32x4 b2 = base2(x.b);
        float part[16];
        static_for<0, 16>([&](auto S) {
          constexpr int s = decltype(S)::value;
          const float dats = sdA[t][s], dast = sdA[s][t];
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ex = exp_nonpos(b2[e], row_bcast<s>(b2[e]));
            const float kx = row_bcast<s>(x.k[e]) * ex;
            dqd[e] += dats * kx;
            acc += x.q[e] * kx;
            dkd[e] += dast * row_bcast<s>(x.q[e]) * ex;
          }
          part[s] = s <= t ? acc : 0.f;
          __builtin_amdgcn_sched_barrier(0);  // one s at a time: bounded register use
        });
        const f32x4 r = reduce_scores(part);
        *reinterpret_cast<f32x4*>(&sRed[w][t][4 * g4]) = r;
      }
      __syncthreads();
      if (!moderate && tid < kSB * kSB) {
        const int tt = tid >> 4, ss = tid & 15;
        float acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < NCB; ++ww) acc += sRed[ww][tt][ss];
        sA[tt * LDA + ss] = (E)acc;
      }
      // ---- dq, dk, dg (channels 16w + 4g4 + i of token n16) ----
      // the global state before the sub-block, rows 16w .. in U's lane layout, rounded to the
      // element type (the MFMA operand type, as the stored chunk states are)
      typename Piece4<E>::type Sj[NJB];
      if (urole) {
        // the stored state before the chunk, advanced through the chunk's earlier sub-blocks
        f32x4 Sf[NJB];
        if (from_store) {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) Sf[jb] = widen(Sc[jb]);
        } else {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb)
            Sf[jb] = load4(a.seg_in + (long)seg * SS + (long)(16 * w + n16) * DV + jb * 16 + 4 * g4);
        }
        for (int i = 0; i < j; ++i) {
          const float le = sLamE[i][16 * w + n16];
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb)
            Sf[jb] = mma_k16<E, true, true>(Sf[jb] * le, sV + i * kSB * LDV + jb * 16, LDV,
                                            sKt + i * kSB * LDQ + 16 * w, LDQ);
        }
        // the carry into the sub-block from the later tokens, rowsum(S_after * U), formed as
        // rowsum(S_j * exp(lam) U) + sum_s k_s * dk_s|U (S_after = exp(lam) S_j + Ktil^T V): the
        // second term from the same U-part of dk that dg subtracts again, so that where the decay is
        // strong the two cancel to float32 rounding, not to the rounding of S
        float ps = 0.f;
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          ps += piece_dot(Sf[jb], U[jb]);
          if constexpr (sizeof(E) == 2) Sj[jb] = to_bf16x4(Sf[jb]);
          else Sj[jb] = Sf[jb];
        }
        ps = sum_over_g4(ps) * sLamE[j][16 * w + n16];
        f32x4 aq = zero4(), ak = zero4();
        if constexpr (sizeof(E) == 2) {
#pragma unroll
          for (int j0 = 0; j0 < NJB; j0 += 2) {
            const int off = n16 * LDV + 16 * j0 + pair_col(g4);
            aq = Mma<bf16>::mma(merge_pair(Sj[j0], Sj[j0 + 1]), *reinterpret_cast<const bf16x8*>(sdO + off), aq);
            ak = Mma<bf16>::mma(merge_pair(to_bf16x4(U[j0]), to_bf16x4(U[j0 + 1])),
                                *reinterpret_cast<const bf16x8*>(sV + j * kSB * LDV + off), ak);
          }
        } else {
#pragma unroll
          for (int j0 = 0; j0 < NJB; ++j0) {
            const f32x4 rs[1] = {Sj[j0]}, ru[1] = {U[j0]};
            aq = mma_regX<1>(aq, rs, sdO + n16 * LDV + j0 * 16);
            ak = mma_regX<1>(ak, ru, sV + (j * kSB + n16) * LDV + j0 * 16);
          }
        }
        f32x4 dqv, dkv, dgv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float du = __expf(x.lam[i] - x.b[i]) * ak[i];  // dk's U part
          dgv[i] = __shfl(ps, (l & ~15) | (4 * g4 + i)) + row_sum16(x.k[i] * du);  // the carry
          dqv[i] = __expf(x.b[i]) * aq[i] + dqd[i];
          dkv[i] = du + dkd[i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dgv[i] += seg_scan_rev_incl<16>(x.q[i] * dqv[i] - x.k[i] * dkv[i]);
        const long go = (ts0 + n16) * DK + 16 * w + 4 * g4;
        store4(dq + go, dqv);
        store4(dk + go, dkv);
        store4(a.dg + go, dgv);
      }
      __syncthreads();  // the partial scores are consumed: U takes their place
      if (urole) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) store4(sU + (16 * w + n16) * LDU + jb * 16 + 4 * g4, U[jb]);
      }
      __syncthreads();
      // ---- dv^T[j][s] = sum_t dO^T[j][t] A^T[s][t] + sum_c U^T[j][c] Ktil[s][c] ----
      for (int jb = w; jb < NJB; jb += NW) {
        f32x4 acc = mma_k16<E, true, true>(zero4(), sdO + jb * 16, LDV, sA, LDA);
        acc = mma<E, true, false>(acc, sU + jb * 16, LDU, sKt + j * kSB * LDQ, LDQ, 0, DK);
        store4(dv + (ts0 + n16) * DV + jb * 16 + 4 * g4, acc);
      }
      // ---- U before the sub-block ----
      if (urole) {
        const float le = sLamE[j][16 * w + n16];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
          U[jb] = mma_k16<E, true, true>(U[jb] * le, sdO + jb * 16, LDV, sQb + j * kSB * LDQ + 16 * w, LDQ);
      }
      if (more) post_moderate(xn);  // every wave has read sMod for this sub-block before its first barrier
      __syncthreads();
    }
  }
  // D = gradient w.r.t. the state entering the segment (from this segment's outputs); with
  // sub-segments the reverse scan over them gives it, with from_in the state-gradient pass
  if (urole && NS == 1 && !a.from_in) {
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
    float* dst = a.seg_dstate + (long)unit * SS;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) store4(dst + (long)(16 * w + n16) * DV + jb * 16 + 4 * g4, U[jb]);
  }
}

template <typename E, int DK, int DV>
struct FwdExactLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const FwdArgs& a = *static_cast<const FwdArgs*>(pa);
    const int n_units = a.BH * a.P * a.S;  // then the re-split pieces' slots
    hipLaunchKernelGGL((fwd_exact_kernel<E, DK, DV, 8>), dim3(n_units + (a.list ? a.R : 0)), dim3(8 * 64), 0, s, a,
                       n_units);
    return hipGetLastError();
  }
};

template <typename E, int DK, int DV>
struct BwdExactLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.BH * a.P * a.S;  // then the re-split pieces' slots
    hipLaunchKernelGGL((bwd_exact_kernel<E, DK, DV, 8>), dim3(n_units + (a.list ? a.R : 0)), dim3(8 * 64), 0, s, a,
                       n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_fwd_exact(int dtype, int dk, int dv) { return lookup_dd<FwdExactLauncher>(dtype, dk, dv); }
launch_fn lookup_bwd_exact(int dtype, int dk, int dv) { return lookup_dd<BwdExactLauncher>(dtype, dk, dv); }

}  // namespace gla
