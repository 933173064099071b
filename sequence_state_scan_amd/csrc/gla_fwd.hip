// Forward kernels: the local chunkwise pass and the cumulative-decay correction.
//
// Chunkwise form of S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t, over a chunk of
// C tokens with in-chunk running log-decay b_t (inclusive) and chunk total lam = b_{C-1}:
//   Qbar = q * exp(b), Kbar = k * exp(-b), Ktil = k * exp(lam - b)
//   O    = [(Qbar Kbar^T) masked to s <= t] V + Qbar S_prev
//   S    = diag(exp(lam)) S_prev + Ktil^T V
// (Kbar = K / Lambda for the intra-chunk part and Ktil = K * Gamma for the state update: the two
// chunk quantities the ZeCO referee report compares in its minor comment 4; with
// Lambda = exp(b) and Gamma = exp(lam - b) both are exact.)
//
// Every chunk tile is staged in LDS once, token-major as it sits in HBM; operands that contract
// over tokens (V^T, Ktil^T) are read with the transposing LDS load.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// One workgroup of NW waves = one (batch*head, segment) unit, all of d_v.  The state S (float32,
// dk x dv) lives in accumulator registers for the whole segment: wave w owns JPW adjacent
// 16-column blocks (jb = JPW w ..), so in bf16 its output tiles leave as 32-column pairs, 16 bytes
// per lane.  After every chunk the state is also written out (chunk_states, element type E, in the
// tiled chunk-state layout; with two blocks per wave the pair of tiles of each 16-row block leaves
// as 1024 contiguous bytes): the local chunk states the correction turns into global ones and the
// backward reads.  A forward-only caller passes no chunk_states, and the instance with KEEP false
// writes none.
//
// A chunk in which some channel decays by more than kFastMinChunkLogDecay stops the unit: its flag
// is set and the exact sub-block kernel (gla_exact.hip) recomputes the whole unit; otherwise the
// flag is cleared at the end.
//
// Per chunk: (1) every 16-lane row takes items of 16 tokens x 8 channels of q, k and g: the gate's
// running sum comes from DPP scans across the 16 lanes (one token each) and the totals of the
// token-block sets meet in LDS, q and k are scaled and every tile is staged in LDS, and the next
// chunk's q, k, g, v are requested into registers;
// (2) the intra-chunk scores; (3) outputs and the state update on MFMA.  The requests of (1) are
// in flight during (2)-(3).
template <typename E, int C, int DK, int DV, int NW, bool KEEP>
__global__ __launch_bounds__(NW * 64) void fwd_local_kernel(FwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  typedef GateTile8<E, C, DK, NW * 64> GT;  // items of q, k, g: 16 tokens x 8 channels
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDQ = lds_ld<E>(DK), LDKT = lds_ld<E>(DK), LDV = lds_ld<E>(DV), LDT = lds_ld<E>(C);
  constexpr int NJB = DV / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, NW);
  constexpr int KS = Mma<E>::KSTEP, NKS = C / KS;
  static_assert(JPW == 1 || NJB % NW == 0, "a wave owns JPW column blocks, or none");

  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];   // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sK[C * LDQ];   // Kbar [s][c]
  __shared__ __attribute__((aligned(16))) E sKt[C * LDKT]; // Ktil [s][c]
  __shared__ __attribute__((aligned(16))) E sV[C * LDV];   // V    [s][j]
  __shared__ __attribute__((aligned(16))) E sA[C * LDT];   // A    [t][s], masked
  __shared__ __attribute__((aligned(16))) float sLamE[DK];  // exp(lam) per channel
  __shared__ __attribute__((aligned(16))) float sTot[GT::NSET * DK];  // per-set gate totals

  const int unit = blockIdx.x;  // (b, h, segment, sub-segment)
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const float* __restrict__ g = a.g;
  E* __restrict__ o = static_cast<E*>(a.o);
  E* __restrict__ cst = static_cast<E*>(a.chunk_states);
  const int NS = a.S, sub = unit % NS, seg = unit / NS;  // sub-segments per segment, this one, its segment
  const int L = a.T / a.P, Ls = L / NS;
  const int nchunks = Ls / C;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L + (long)sub * Ls;
  const long chunk0 = tok0 / C;  // global chunk index of the sub-segment's first chunk
  const int w = wave_id();
  typedef typename Mma<E>::frag frag;

  // the gate tile of q, k, g (the 16 lanes of a row hold 16 consecutive tokens of 8 channels: their
  // 16-byte LDS writes hit 16 consecutive rows, no bank conflicts)
  GT pgt;
  Vec8<E> pv[VPT];
  auto prefetch = [&](int n, int tid) {
    const long t0 = tok0 + (long)n * C;
    pgt.load(g, q, k, t0 * DK, tid);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pv[i].load(v + (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
  };

  f32x4 S[JPW][NKB];  // S[jj][kb][i] = S[16kb + 4g4 + i][16jb + n16]
  if (a.init && (sub > 0 || a.from_in) && w * JPW < NJB) {
    // the state entering the sub-segment (from its segment's start, or the global one with
    // from_in), row-major float32: each lane reads 4 consecutive columns of a row and the quad
    // transpose turns them into its rows
    const float* ci = a.init + (long)unit * DK * DV;
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        S[jj][kb] = quad_transpose(load4(ci + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + (w * JPW + jj) * 16 + (n16 & ~3)));
  } else {
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) S[jj][kb] = zero4();
  }
  float ldsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // log cumulative decay of the segment (set 0, n16 == 0)

  prefetch(0, threadIdx.x);
  for (int n = 0; n < nchunks; ++n) {
    const long t0 = tok0 + (long)n * C;
    const int tid = fresh_tid(), l = tid & 63, n16 = l & 15, g4 = l >> 4;
    // ---- (1) gate prefix sums, Qbar, Kbar, Ktil, V -> LDS; request the next chunk ----
    int strong = 0;  // a channel decays by more than the factorisation takes in this chunk
    {
      float b[GT::RI][8], lam[8];
      pgt.prefix(tid, sTot, b, lam);
      if (GT::active(tid)) {
        const int x = GT::group_of(tid);
        float el[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          el[e] = __expf(lam[e]);
          strong |= lam[e] < kFastMinChunkLogDecay;
        }
#pragma unroll
        for (int r = 0; r < GT::RI; ++r) {
          float xq[8], xk[8], xkt[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float eb = __expf(b[r][e]);
            xq[e] = pgt.q[r].at(e) * eb;
            xk[e] = pgt.k[r].at(e) * __builtin_amdgcn_rcpf(eb);  // exp(-b) to one ulp
            xkt[e] = xk[e] * el[e];
          }
          const int row = GT::row(tid, r);
          store8(sQ + row * LDQ + 8 * x, xq);
          store8(sK + row * LDQ + 8 * x, xk);
          store8(sKt + row * LDKT + 8 * x, xkt);
        }
        if (GT::set_of(tid) == 0 && n16 == 0) {
          store8(sLamE + 8 * x, el);
#pragma unroll
          for (int e = 0; e < 8; ++e) ldsum[e] += lam[e];
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int pc = tid + NT * i;
        if (NVP % NT == 0 || pc < NVP) pv[i].store(sV + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the next chunk's loads after this chunk's staging
    if (n + 1 < nchunks) prefetch(n + 1, tid);
    if (__syncthreads_or(strong)) {  // the exact sub-block kernel redoes this unit
      if (threadIdx.x == 0) a.flags[unit] = 1;
      return;
    }
    // ---- (2) intra-chunk scores: A^T[s][t] = Kbar[s] . Qbar[t], kept for s <= t, stored as A[t][s] ----
    for (int idx = w; idx < NTT * NTT; idx += NW) {
      const int sT = idx / NTT, tT = idx - (idx / NTT) * NTT;
      f32x4 acc = zero4();
      if (sT <= tT) acc = mma<E, false, false>(acc, sK + sT * 16 * LDQ, LDQ, sQ + tT * 16 * LDQ, LDQ, 0, DK);
      const int t = tT * 16 + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (sT * 16 + 4 * g4 + i > t) acc[i] = 0.f;
      store4(sA + t * LDT + sT * 16 + 4 * g4, acc);
    }
    __syncthreads();
    // ---- (3) outputs O^T[j][t] = V^T A^T + S_prev^T Qbar^T, then the state update ----
    // Every operand fragment is read from LDS once per chunk: V^T of the wave's column blocks
    // serves the intra-chunk outputs and the state update; each A, Qbar and Ktil^T fragment
    // serves all of the wave's column blocks.
    if (w * JPW < NJB) {
      E* const cs = KEEP ? cst + (chunk0 + n) * (long)DK * DV : nullptr;
      frag fv[JPW][NKS];
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) fv[jj][ks] = frag_ld<E, true>(sV + (w * JPW + jj) * 16, LDV, ks * KS);
      f32x4 acc[JPW][NTT];
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) acc[jj][tT] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          if (ks * KS < (tT + 1) * 16) {  // tokens s <= t only
            const frag fa = frag_ld<E, false>(sA + tT * 16 * LDT, LDT, ks * KS);
#pragma unroll
            for (int jj = 0; jj < JPW; ++jj) acc[jj][tT] = Mma<E>::mma(fv[jj][ks], fa, acc[jj][tT]);
          }
      }
      if constexpr (sizeof(E) == 2) {
        static_assert(NKB % 2 == 0, "d_k a multiple of 32");
#pragma unroll
        for (int pp = 0; pp < NKB / 2; ++pp) {
          // merged, the lane's pieces of blocks 2pp and 2pp + 1 are the 8 adjacent rows
          // 32 pp + pair_col(g4) + 0..7 of S: the Qbar fragment is one 16-byte read
          bf16x8 x[JPW];
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) x[jj] = merge_pair(to_bf16x4(S[jj][2 * pp]), to_bf16x4(S[jj][2 * pp + 1]));
#pragma unroll
          for (int tT = 0; tT < NTT; ++tT) {
            const bf16x8 y = *reinterpret_cast<const bf16x8*>(sQ + (tT * 16 + n16) * LDQ + 32 * pp + pair_col(g4));
#pragma unroll
            for (int jj = 0; jj < JPW; ++jj) acc[jj][tT] = Mma<bf16>::mma(x[jj], y, acc[jj][tT]);
          }
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) mma_regX_rows<NKB, NTT>(acc[jj], S[jj], sQ + n16 * LDQ, 16 * LDQ);
      }
      if constexpr (sizeof(E) == 2 && JPW == 2) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT)
          *reinterpret_cast<bf16x8*>(o + (t0 + tT * 16 + n16) * DV + w * 32 + pair_col(g4)) =
              merge_pair(to_bf16x4(acc[0][tT]), to_bf16x4(acc[1][tT]));
      } else {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
          for (int tT = 0; tT < NTT; ++tT)
            store4(o + (t0 + tT * 16 + n16) * DV + (w * JPW + jj) * 16 + 4 * g4, acc[jj][tT]);
      }
      // S = diag(exp(lam)) S + Ktil^T V
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4 lamE = load4(sLamE + kb * 16 + 4 * g4);
        frag fk[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) fk[ks] = frag_ld<E, true>(sKt + kb * 16, LDKT, ks * KS);
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          S[jj][kb] *= lamE;
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) S[jj][kb] = Mma<E>::mma(fk[ks], fv[jj][ks], S[jj][kb]);
        }
        if constexpr (!KEEP) continue;  // a forward-only caller keeps no per-chunk states
        if constexpr (JPW == 2) {  // the wave's two blocks are a pair of the tiled layout
          store_state_pair<E, NJB>(cs, kb, w, state_lane_qt(n16, g4), quad_transpose(S[0][kb]),
                                   quad_transpose(S[1][kb]));
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            store_state_piece<E, NJB>(cs, kb, w * JPW + jj, state_lane_qt(n16, g4), quad_transpose(S[jj][kb]));
        }
      }
    }
    __syncthreads();
  }

  // ---- segment results: local end state (float32) and log cumulative decay (with from_in the
  // state pass has given them) ----
  const int tid = threadIdx.x;
  if (a.from_in) {
  } else if (NS == 1) {
    float* st = a.seg_state + (long)unit * DK * DV;
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w * JPW + jj;
      if (w * JPW < NJB)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          store4(st + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + jb * 16 + (n16 & ~3), quad_transpose(S[jj][kb]));
    }
    if (GT::active(tid) && GT::set_of(tid) == 0 && (tid & 15) == 0)
      store8(a.seg_logdecay + (long)unit * DK + 8 * GT::group_of(tid), ldsum);
  } else if (sub == NS - 1) {
    // the segment's end state comes from the scan over its sub-segments; its log decay is the sum
    // of the sub-segments' (from the state pass)
    for (int c = tid; c < DK; c += NT) {
      float sum = 0.f;
      for (int s2 = 0; s2 < NS; ++s2) sum += a.sub_ld[((long)seg * NS + s2) * DK + c];
      a.seg_logdecay[(long)seg * DK + c] = sum;
    }
  }
  if (tid == 0) a.flags[unit] = 0;
}

// State pass over sub-segments: the state at the end of every sub-segment from a zero start,
// S = diag(exp(lam)) S + Ktil^T V per chunk (no outputs), and the sub-segment's summed log-gates.
// Every factor is exp(<= 0), so no chunk needs the exact kernels here.  Layout and per-chunk
// staging as in fwd_local_kernel; only k, g and v are read.
// With a.reach the same end state is summed from the other side: the chunks from the last one
// back, S += Khat^T V with Khat_t = k_t exp(x_t), x_t the log-gates after token t up to the
// sub-segment's end (lam - b_t plus the later chunks' totals), and no decay of S.  Once every
// channel's running total is below kReachCut the earlier chunks' Khat are exact zeros and the
// walk stops; the log-gate output is then the total of the chunks walked, itself below the cut,
// so that its exponential is the same 0.0f.
template <typename E, int C, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_state_kernel(FwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  typedef GateTile8<E, C, DK, NW * 64> GT;
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDKT = lds_ld<E>(DK), LDV = lds_ld<E>(DV);
  constexpr int NJB = DV / 16, NKB = DK / 16;
  constexpr int JPW = ceil_div(NJB, NW);
  constexpr int KS = Mma<E>::KSTEP, NKS = C / KS;
  static_assert(JPW == 1 || NJB % NW == 0, "a wave owns JPW column blocks, or none");

  __shared__ __attribute__((aligned(16))) E sKt[C * LDKT];  // Ktil [s][c]
  __shared__ __attribute__((aligned(16))) E sV[C * LDV];    // V    [s][j]
  __shared__ __attribute__((aligned(16))) float sLamE[DK];
  __shared__ __attribute__((aligned(16))) float sTot[GT::NSET * DK];

  __shared__ int sList[NT / 64];
  __shared__ int sLive[2 * NW];  // the reach walk's stop vote
  UnitPlace up;
  if (a.list) {  // the re-split: list the flagged units (workgroup 0 writes the list), then this piece
    int n, X;
    const int u = resplit_derive<NT>(a.flags, a.BH * a.P * a.S, a.R, a.xmax, blockIdx.x, blockIdx.x == 0 ? a.list : nullptr,
                                     sList, n, X);
    up = u >= 0 ? list_place(a, blockIdx.x, X, u, DK, (long)DK * DV) : UnitPlace{};
  } else {
    up = unit_place(a, n_units, DK, (long)DK * DV);
  }
  if (!up.live || up.X == 1) return;  // a whole re-split unit has no pieces to combine
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const int S = up.NS, sub = up.sub, seg = up.seg;
  const int L = a.T / a.P, Ls = L / S, nchunks = Ls / C;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L + (long)sub * Ls;
  const int w = wave_id();
  typedef typename Mma<E>::frag frag;

  GT pgt;
  Vec8<E> pv[VPT];
  auto prefetch = [&](int n, int tid) {
    const long t0 = tok0 + (long)n * C;
    pgt.load(a.g, nullptr, k, t0 * DK, tid);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pv[i].load(v + (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
  };

  f32x4 S_[JPW][NKB];
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) S_[jj][kb] = zero4();
  // the summed log-gates of the chunks walked so far (every active lane, for its 8 channels)
  float ldsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // reach: walk from the last chunk, token t weighted by exp(log-gates after t), no decay of S;
  // stop once every channel is past kReachCut
  const bool reach = a.reach && !a.list;

  prefetch(reach ? nchunks - 1 : 0, threadIdx.x);
  for (int it = 0; it < nchunks; ++it) {
    const int n = reach ? nchunks - 1 - it : it;
    const int tid = fresh_tid(), l = tid & 63, n16 = l & 15, g4 = l >> 4;
    {
      float b[GT::RI][8], lam[8];
      pgt.prefix(tid, sTot, b, lam);
      if (GT::active(tid)) {
        const int x = GT::group_of(tid);
        float after[8];  // log-gates after the chunk (reach), else 0
#pragma unroll
        for (int e = 0; e < 8; ++e) after[e] = reach ? ldsum[e] : 0.f;
#pragma unroll
        for (int r = 0; r < GT::RI; ++r) {
          float xkt[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xkt[e] = pgt.k[r].at(e) * __expf(lam[e] - b[r][e] + after[e]);
          store8(sKt + GT::row(tid, r) * LDKT + 8 * x, xkt);
        }
        if (!reach && GT::set_of(tid) == 0 && n16 == 0) {
          float el[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) el[e] = __expf(lam[e]);
          store8(sLamE + 8 * x, el);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ldsum[e] += lam[e];
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int pc = tid + NT * i;
        if (NVP % NT == 0 || pc < NVP) pv[i].store(sV + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < nchunks) prefetch(reach ? n - 1 : n + 1, tid);
    __syncthreads();
    if (w * JPW < NJB) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        frag fk[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) fk[ks] = frag_ld<E, true>(sKt + kb * 16, LDKT, ks * KS);
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          if (!reach) S_[jj][kb] *= load4(sLamE + kb * 16 + 4 * g4);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            S_[jj][kb] = Mma<E>::mma(fk[ks], frag_ld<E, true>(sV + (w * JPW + jj) * 16, LDV, ks * KS), S_[jj][kb]);
        }
      }
    }
    if (reach) {
      bool live = false;  // some channel of this lane's item still above the cut
      if (GT::active(tid))
#pragma unroll
        for (int e = 0; e < 8; ++e) live |= ldsum[e] >= kReachCut;
      if (!barrier_any<NW>(sLive, it & 1, live)) break;
    } else {
      __syncthreads();
    }
  }
  float* st = up.st;
  const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
  if (w * JPW < NJB) {
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        store4(st + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + (w * JPW + jj) * 16 + (n16 & ~3),
               quad_transpose(S_[jj][kb]));
  }
  const int tid = threadIdx.x;
  if (GT::active(tid) && GT::set_of(tid) == 0 && (tid & 15) == 0)
    store8(up.ld + 8 * GT::group_of(tid), ldsum);
}

// Correction of segment p's local results with its incoming global state S_in[p]:
//   o_t              += (q_t * a_t) . S_in[p],   a_t = exp(sum of g from the segment start to t)
//   chunk_states[n]  += diag(a at the end of chunk n) S_in[p]    (unless no chunk states are kept)
// With g <= 0, a_t only decreases: once every a_t of a chunk is exactly 0.0f, so are all later
// ones (and the chunk-end decays), and the loop stops.
//
// SPLIT: a segment is cut into a.S sub-segments of consecutive chunks, one workgroup each.  The
// workgroup of a later sub-segment first walks the gate of the chunks before it, with the same
// prefix sums in the same order as the one-workgroup walk, so its running sums, its early stop and
// so its results are bit for bit those of the walk over the whole segment.  Workgroups are
// numbered sub-segment first, so that the first sub-segments of every segment, where the
// correction is live, are dispatched first.
//
// One workgroup of NW waves per unit.  S_in is constant over the segment: wave w owns the JPW
// adjacent d_v column blocks JPW w.., held in fp32 registers in the store layout (4 consecutive
// j of one row c) for S_n += a_end S_in, and S_in^T sits in LDS in the element type as the MFMA
// operand of o += (q * a) S_in, each fragment read once per chunk for all token tiles.  Per live
// chunk every read (g, q, o, the chunk state) is issued first; o moves as merged pairs of
// 16-column tiles (16 bytes per lane) in bf16; q * a goes to LDS, double-buffered by chunk parity,
// so that besides the gate tile's set exchange one barrier per chunk suffices.
template <typename E, int C, int DK, int DV, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void correct_fwd_kernel(CorrArgs a, int n_units) {
  typedef GateTile8<E, C, DK, NW * 64> GT;  // items of g and q: 16 tokens x 8 channels
  constexpr int LDQ = lds_ld<E>(DK), LDR = lds_ld<E>(DK);
  constexpr int NJB = DV / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, NW);
  constexpr bool PAIRS = sizeof(E) == 2 && JPW == 2;  // output tiles leave as merged pairs
  static_assert(JPW == 1 || NJB % NW == 0, "a wave owns JPW column blocks, or none");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sRT[DV * LDR];   // S_in^T  [j][c]
  __shared__ __attribute__((aligned(16))) E sQ[2][C * LDQ];  // q * a   [t][c]
  __shared__ float sAend[2][DK];                              // a at the chunk's last token
  __shared__ __attribute__((aligned(16))) float sTot[GT::NSET * DK];  // per-set gate totals

  const int unit = blockIdx.x;
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const float* __restrict__ g = a.g;
  E* __restrict__ o = static_cast<E*>(a.o);
  E* __restrict__ cst = static_cast<E*>(a.chunk_states);
  const int NS = SPLIT ? a.S : 1, nseg = a.BH * a.P;  // sub-segments per segment, segments
  const int sub = SPLIT ? unit / nseg : 0, seg = SPLIT ? unit - sub * nseg : unit;
  const int L = a.T / a.P;
  const int nchunks = L / C, nsub = nchunks / NS;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const long chunk0 = (long)seg * nchunks;
  constexpr long SS = (long)DK * DV;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool vrole = w * JPW < NJB;  // owns the column blocks JPW w ..
  const int x8 = GT::group_of(tid);

  // ST[jj][kb][i] = S_in[16kb + 4g4 + (n16&3)][16jb + (n16&~3) + i]  (store layout, fp32);
  // its quad transpose, S_in[16kb + 4g4 + i][16jb + n16], is 4 consecutive c of row j of S_in^T
  const float* sin = a.seg_in + (long)seg * SS;
  f32x4 ST[JPW][NKB];
  int nonzero = 0;
  if (vrole) {
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w * JPW + jj;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        ST[jj][kb] = load4(sin + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + jb * 16 + (n16 & ~3));
        store4(sRT + (jb * 16 + n16) * LDR + kb * 16 + 4 * g4, quad_transpose(ST[jj][kb]));
#pragma unroll
        for (int i = 0; i < 4; ++i) nonzero |= ST[jj][kb][i] != 0.f;
      }
    }
  }
  if (!__syncthreads_or(nonzero)) return;  // zero incoming state: nothing to add

  float carry[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // sum of g from the segment start to the previous chunk's end
  // the gate of the chunks before the sub-segment, NB chunks' loads in flight at a time
  constexpr int NB = 4;
  if constexpr (SPLIT) {
    for (int n0 = 0; n0 < sub * nsub; n0 += NB) {
      GT pg[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (n0 + i < sub * nsub) pg[i].load(g, nullptr, nullptr, (tok0 + (long)(n0 + i) * C) * DK, tid);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (n0 + i < sub * nsub) {
          float b[GT::RI][8], lam[8];
          pg[i].prefix(tid, sTot, b, lam);
          int live = 0;
          if (GT::active(tid)) {
#pragma unroll
            for (int r = 0; r < GT::RI; ++r)
#pragma unroll
              for (int e = 0; e < 8; ++e) live |= __expf(carry[e] + b[r][e]) != 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) carry[e] += lam[e];
          }
          if (!__syncthreads_or(live)) return;  // the walk stops before the sub-segment
        }
      }
    }
  }
  for (int n = sub * nsub; n < (sub + 1) * nsub; ++n) {
    const long t0 = tok0 + (long)n * C;
    const int par = n & 1;
    E* const cs = cst ? cst + (chunk0 + n) * SS : nullptr;  // null: a forward-only caller keeps no chunk states
    // ---- every read of the chunk first ----
    GT pgt;
    pgt.load(g, q, nullptr, t0 * DK, tid);
    piece oprev[JPW][NTT], cprev[JPW][NKB];
    if (vrole) {
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) {
        if constexpr (PAIRS) {
          unmerge_pair(*reinterpret_cast<const bf16x8*>(o + (t0 + tT * 16 + n16) * DV + w * 32 + pair_col(g4)),
                       oprev[0][tT], oprev[1][tT]);
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            oprev[jj][tT] = load_piece(o + (t0 + tT * 16 + n16) * DV + (w * JPW + jj) * 16 + 4 * g4);
        }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (!cs) break;
        if constexpr (JPW == 2) {
          load_state_pair<E, NJB>(cs, kb, w, state_lane_qt(n16, g4), cprev[0][kb], cprev[1][kb]);
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            cprev[jj][kb] = load_state_piece<E, NJB>(cs, kb, w * JPW + jj, state_lane_qt(n16, g4));
        }
      }
    }
    // ---- a_t = exp(sum of g from the segment start to t); q * a -> LDS ----
    int live = 0;
    {
      float b[GT::RI][8], lam[8];
      pgt.prefix(tid, sTot, b, lam);
      if (GT::active(tid)) {
#pragma unroll
        for (int r = 0; r < GT::RI; ++r) {
          float xq[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float av = __expf(carry[e] + b[r][e]);
            live |= av != 0.f;
            xq[e] = pgt.q[r].at(e) * av;
          }
          store8(&sQ[par][GT::row(tid, r) * LDQ + 8 * x8], xq);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) carry[e] += lam[e];
        if (GT::set_of(tid) == 0 && n16 == 0) {
          float ae[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) ae[e] = __expf(carry[e]);
          store8(&sAend[par][8 * x8], ae);
        }
      }
    }
    if (!__syncthreads_or(live)) break;  // every a_t of this chunk (and all later ones) is 0
    if (vrole) {
      // o^T[j][t] += sum_c S_in^T[j][c] (q_t a_t)[c]
      f32x4 acc[JPW][NTT];
#pragma unroll
      for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) acc[jj][tT] = widen(oprev[jj][tT]);
#pragma unroll
      for (int kk = 0; kk < DK; kk += Mma<E>::KSTEP) {
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj) {
          const typename Mma<E>::frag x = frag_ld<E, false>(sRT + (w * JPW + jj) * 16 * LDR, LDR, kk);
#pragma unroll
          for (int tT = 0; tT < NTT; ++tT)
            acc[jj][tT] = Mma<E>::mma(x, frag_ld<E, false>(&sQ[par][tT * 16 * LDQ], LDQ, kk), acc[jj][tT]);
        }
      }
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) {
        if constexpr (PAIRS) {
          *reinterpret_cast<bf16x8*>(o + (t0 + tT * 16 + n16) * DV + w * 32 + pair_col(g4)) =
              merge_pair(to_bf16x4(acc[0][tT]), to_bf16x4(acc[1][tT]));
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) store4(o + (t0 + tT * 16 + n16) * DV + (w * JPW + jj) * 16 + 4 * g4, acc[jj][tT]);
        }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if (!cs) break;
        const float ae = sAend[par][kb * 16 + 4 * g4 + (n16 & 3)];
        if constexpr (JPW == 2) {
          store_state_pair<E, NJB>(cs, kb, w, state_lane_qt(n16, g4), widen(cprev[0][kb]) + ae * ST[0][kb],
                                   widen(cprev[1][kb]) + ae * ST[1][kb]);
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            store_state_piece<E, NJB>(cs, kb, w * JPW + jj, state_lane_qt(n16, g4), widen(cprev[jj][kb]) + ae * ST[jj][kb]);
        }
      }
    }
  }
}

template <typename E, int C, int DK, int DV>
struct FwdLocalLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const FwdArgs& a = *static_cast<const FwdArgs*>(pa);
    const int n_units = a.BH * a.P * a.S;
    if (a.chunk_states)
      hipLaunchKernelGGL((fwd_local_kernel<E, C, DK, DV, 8, true>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    else
      hipLaunchKernelGGL((fwd_local_kernel<E, C, DK, DV, 8, false>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};

template <typename E, int C, int DK, int DV>
struct FwdStateLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const FwdArgs& a = *static_cast<const FwdArgs*>(pa);
    const int n_units = a.list ? 0 : a.BH * a.P * a.S;  // the units, or the re-split pieces' slots
    hipLaunchKernelGGL((fwd_state_kernel<E, C, DK, DV, 8>), dim3(a.list ? a.R : n_units), dim3(8 * 64), 0, s, a,
                       n_units);
    return hipGetLastError();
  }
};

template <typename E, int C, int DK, int DV>
struct CorrectFwdLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P * a.S;
    if (a.S > 1)
      hipLaunchKernelGGL((correct_fwd_kernel<E, C, DK, DV, 8, true>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    else
      hipLaunchKernelGGL((correct_fwd_kernel<E, C, DK, DV, 8, false>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_fwd_local(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<FwdLocalLauncher>(dtype, chunk, dk, dv);
}
launch_fn lookup_fwd_state(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<FwdStateLauncher>(dtype, chunk, dk, dv);
}
launch_fn lookup_correct_fwd(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<CorrectFwdLauncher, Bf16CorrChunks>(dtype, chunk, dk, dv);
}

}  // namespace gla
