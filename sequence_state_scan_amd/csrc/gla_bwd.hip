// Backward of the chunkwise form, per segment, given the GLOBAL state after every chunk
// (chunk_states, written by the local pass and corrected by the forward correction) and the
// segment's global incoming state S_in.  With b, lam, Qbar, Kbar as in the forward, per chunk n:
//   dA[t][s] = do_t . v_s  for s <= t,    A = (Qbar Kbar^T) masked the same way
//   dq       = exp(b) * (dO S_{n-1}^T + dA Kbar)                      (global)
//   dk       = exp(-b) * (dA^T Qbar + V (exp(lam) U_n)^T)             U_n: dL/dS after chunk n
//   dv       = A^T dO + Kbar (exp(lam) U_n)
//   U_{n-1}  = exp(lam) U_n + Qbar^T dO                               (U starts at 0: local)
//   dg_t     = sum_{t <= t' in chunk n} (q dq - k dk)_t' + rowsum(S_n * U_n)
// The last line is exact: over the segment's tokens after chunk n the running sum of
// q dq - k dk equals rowsum(S_n * U_n) (the closed form of dg applied to that suffix), so no sum
// ever runs over more than one chunk.  The carry is formed inside the chunk, as
// rowsum(S_{n-1} * exp(lam) U_n) + sum_s (k dk|U_n)_s with dk|U_n the U_n part of dk (the two
// pieces of S_n = exp(lam) S_{n-1} + Ktil^T V), not from the stored S_n: the suffix sum subtracts
// the same U_n terms again, so where the decay is strong (S_n made of the chunk's own last tokens)
// they cancel to float32 rounding rather than to the stored state's rounding.
//
// A chunk in which some channel decays by more than kFastMinChunkLogDecay stops the unit: its flag
// is set and the exact sub-block kernel (gla_exact.hip) recomputes the whole unit.
//
// One workgroup of NW waves walks each segment from its end.  Wave w keeps the 16 rows
// c = 16w.. of U^T (all of d_v) in accumulator registers: they feed dq and dk, which contract U
// and the chunk state over d_v.  dv contracts U over d_k instead, so once per chunk the waves
// write exp(lam) U into LDS (as rows U[c][:], half of d_v at a time), and dv's tiles read it
// back with the transposing load.  q, k, g, v and do are read from HBM once per chunk (q, k, g as
// gate tiles of 16 tokens x 8 channels); the chunk state arrives in U's lane layout, a pair of
// tiles of the tiled chunk-state layout per 16-byte load; dq, dk and dv leave as merged pairs of
// 16-column tiles, 16 bytes per lane.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// Value of x at the first lane of the 16-lane row, on every lane of the row.
__device__ __forceinline__ float row_first(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150, 0xF, 0xF, false));  // row_newbcast:0
}

template <typename E, int C, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_kernel(BwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  typedef GateTile8<E, C, DK, NW * 64> GT;  // items of q, k, g: 16 tokens x 8 channels
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDV = lds_ld<E>(DV), LDQ = lds_ld<E>(DK), LDK = lds_ld_frag<E>(DK), LDT = lds_ld<E>(C);
  constexpr int DVH = DV < 128 ? DV : 128, NH = DV / DVH;  // d_v columns of U staged at a time
  constexpr int LDU = lds_ld<E>(DVH);
  constexpr int NJB = DV / 16, NCB = DK / 16, NTT = C / 16, NJH = DVH / 16;
  constexpr int KS = Mma<E>::KSTEP;
  constexpr int KU = sizeof(E) == 2 ? 2 : 1;  // 16-wide d_v blocks per k-step of the MFMA
  static_assert(NCB <= NW, "one 16-row block of U^T per wave");
  static_assert(NJB % KU == 0, "d_v blocks pair up for bf16");
  static_assert(NW % NTT == 0, "the waves split evenly over the chunk's 16-token blocks");
  typedef typename Piece4<E>::type piece;

  // LDS.  sV and sLam are dead once dq / dk are done; the U staging area then reuses them.
  constexpr int SZ_V = C * LDV * (int)sizeof(E), SZ_Q = C * LDQ * (int)sizeof(E), SZ_K = C * LDK * (int)sizeof(E),
                SZ_T = C * LDT * (int)sizeof(E);
  constexpr int SZ_U = DK * LDU * (int)sizeof(E);
  constexpr int SZ_VL = SZ_V + SZ_Q > SZ_U ? SZ_V + SZ_Q : SZ_U;  // V and exp(b), later the U staging
  constexpr int OFF_DO = 0, OFF_V = OFF_DO + SZ_V, OFF_LAM = OFF_V + SZ_V, OFF_Q = OFF_V + SZ_VL,
                OFF_K = OFF_Q + SZ_Q, OFF_DAT = OFF_K + SZ_K, OFF_AT = OFF_DAT + SZ_T, SMEM = OFF_AT + SZ_T;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  __shared__ __attribute__((aligned(16))) float sLamE[DK];
  __shared__ __attribute__((aligned(16))) float sTot[GT::NSET * DK];  // per-set gate totals
  E* const sdO = reinterpret_cast<E*>(smem + OFF_DO);    // dO   [t][j]
  E* const sV = reinterpret_cast<E*>(smem + OFF_V);      // V    [s][j]
  E* const sU = reinterpret_cast<E*>(smem + OFF_V);      // exp(lam) U [c][j - half start], after dq / dk
  E* const sLam = reinterpret_cast<E*>(smem + OFF_LAM);  // exp(b) [t][c]
  E* const sQ = reinterpret_cast<E*>(smem + OFF_Q);      // Qbar [t][c]
  E* const sK = reinterpret_cast<E*>(smem + OFF_K);      // Kbar [s][c]
  E* const sdAT = reinterpret_cast<E*>(smem + OFF_DAT);  // dA^T [s][t], masked
  E* const sAT = reinterpret_cast<E*>(smem + OFF_AT);    // A^T  [s][t], masked

  const int unit = blockIdx.x;
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const E* __restrict__ dO = static_cast<const E*>(a.dO);
  const E* __restrict__ cst = static_cast<const E*>(a.chunk_states);
  const float* __restrict__ g = a.g;
  E* __restrict__ dq = static_cast<E*>(a.dq);
  E* __restrict__ dk = static_cast<E*>(a.dk);
  E* __restrict__ dv = static_cast<E*>(a.dv);
  float* __restrict__ dg = a.dg;
  const int NS = a.S, sub = unit % NS, seg = unit / NS;  // sub-segments per segment, this one, its segment
  const int L = a.T / a.P, Ls = L / NS;
  const int nchunks = Ls / C;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L + (long)sub * Ls;
  const long chunk0 = tok0 / C;  // global chunk index of the sub-segment's first chunk
  constexpr long SS = (long)DK * DV;  // one state
  const int w = wave_id();
  const int cb = w;                   // this wave's 16-row block of U^T (waves w >= NCB hold none)
  const bool urole = cb < NCB;

  // the gate tile of q, k, g (the 16 lanes of a row hold 16 consecutive tokens of 8 channels: their
  // 16-byte LDS writes hit 16 consecutive rows, no bank conflicts)
  GT pgt;
  auto prefetch = [&](int n, int tid) { pgt.load(g, q, k, (tok0 + (long)n * C) * DK, tid); };

  // V and dO of a chunk, requested at the chunk's start
  Vec8<E> pv[VPT], pd[VPT];
  auto prefetch_vd = [&](int n, int tid) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) {
        const long off = (tok0 + (long)n * C + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8;
        pv[i].load(v + off);
        pd[i].load(dO + off);
      }
    }
  };

  f32x4 U[NJB];  // U[jb][i] = U[16cb + n16][16jb + 4g4 + i]
  if (a.init && (sub < NS - 1 || a.from_in) && urole) {
    // the gradient w.r.t. the state leaving the sub-segment (from the rest of its segment, or the
    // global one with from_in)
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
      U[jb] = load4(a.init + (long)unit * SS + (long)(cb * 16 + n16) * DV + jb * 16 + 4 * g4);
  } else {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) U[jb] = zero4();
  }

  prefetch(nchunks - 1, threadIdx.x);
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    const int tid = fresh_tid(), l = tid & 63, n16 = l & 15, g4 = l >> 4;
    prefetch_vd(n, tid);  // this chunk's V and dO
    // ---- (1) gate prefix sums, Qbar, Kbar, exp(b); V, dO -> LDS ----
    int strong = 0;  // a channel decays by more than the factorisation takes in this chunk
    {
      float b[GT::RI][8], lam[8];
      pgt.prefix(tid, sTot, b, lam);
      if (GT::active(tid)) {
        const int x = GT::group_of(tid);
#pragma unroll
        for (int e = 0; e < 8; ++e) strong |= lam[e] < kFastMinChunkLogDecay;
#pragma unroll
        for (int r = 0; r < GT::RI; ++r) {
          float xq[8], xk[8], eb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            eb[e] = __expf(b[r][e]);
            xq[e] = pgt.q[r].at(e) * eb[e];
            xk[e] = pgt.k[r].at(e) * __builtin_amdgcn_rcpf(eb[e]);  // exp(-b) to one ulp
          }
          const int off = GT::row(tid, r) * LDQ + 8 * x;
          store8(sQ + off, xq);
          store8(sK + GT::row(tid, r) * LDK + 8 * x, xk);
          store8(sLam + off, eb);
        }
        if (GT::set_of(tid) == 0 && n16 == 0) {
          float el[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) el[e] = __expf(lam[e]);
          store8(sLamE + 8 * x, el);
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int pc = tid + NT * i;
        if (NVP % NT == 0 || pc < NVP) {
          const int off = (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8;
          pv[i].store(sV + off);
          pd[i].store(sdO + off);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (n > 0) prefetch(n - 1, tid);
    // the global state before this chunk, in U's lane layout (read during (2), used in (3))
    piece Sp[NJB];
    if (urole) {
      const long roff = (long)(cb * 16 + n16) * DV + 4 * g4;
      if (n > 0 || sub > 0) {  // the stored global state after the previous chunk
        const E* st = cst + (chunk0 + n - 1) * SS;
        if constexpr (NJB % 2 == 0) {
#pragma unroll
          for (int m = 0; m < NJB / 2; ++m)
            load_state_pair<E, NJB>(st, cb, m, state_lane_row(n16, g4), Sp[2 * m], Sp[2 * m + 1]);
        } else {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb) Sp[jb] = load_state_piece<E, NJB>(st, cb, jb, state_lane_row(n16, g4));
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const f32x4 x = load4(a.seg_in + (long)seg * SS + roff + jb * 16);  // the segment's incoming state
#pragma unroll
          for (int i = 0; i < 4; ++i) Sp[jb][i] = (E)x[i];
        }
      }
    }
    if (__syncthreads_or(strong)) {  // the exact sub-block kernel redoes this unit
      if (threadIdx.x == 0) a.flags[unit] = 1;
      return;
    }
    // ---- (2) dA[t][s] = dO[t] . V[s] and A[t][s] = Qbar[t] . Kbar[s], stored transposed, s <= t.
    // The tiles with sT <= tT are dealt to the waves longest first (the dA tiles contract over d_v,
    // the A tiles over d_k) in snake order, so the SIMDs get about the same MFMA work; the all-zero
    // tiles above the diagonal are only stored. ----
    {
      constexpr int NLT = NTT * (NTT + 1) / 2, NUT = NTT * (NTT - 1) / 2;
      for (int i = 0;; ++i) {
        const int slot = i * NW + ((i & 1) ? NW - 1 - w : w);
        if (slot >= 2 * NLT) break;
        const bool isA = slot >= NLT;
        int j = isA ? slot - NLT : slot, tT = 0;  // j-th tile of the lower triangle, row-major
        while (j > tT) j -= ++tT;
        const int sT = j;
        f32x4 acc = zero4();
        if (isA) acc = mma<E, false, false>(acc, sQ + tT * 16 * LDQ, LDQ, sK + sT * 16 * LDK, LDK, 0, DK);
        else acc = mma<E, false, false>(acc, sdO + tT * 16 * LDV, LDV, sV + sT * 16 * LDV, LDV, 0, DV);
        const int s = sT * 16 + n16;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (tT * 16 + 4 * g4 + q < s) acc[q] = 0.f;
        store4((isA ? sAT : sdAT) + s * LDT + tT * 16 + 4 * g4, acc);
      }
      for (int z = w; z < 2 * NUT; z += NW) {
        const bool isA = z >= NUT;
        int j = isA ? z - NUT : z, tT = 0;  // j-th tile strictly above the diagonal
        while (j >= NTT - 1 - tT) j -= NTT - 1 - tT++;
        const int sT = tT + 1 + j;
        store4((isA ? sAT : sdAT) + (sT * 16 + n16) * LDT + tT * 16 + 4 * g4, zero4());
      }
    }
    __syncthreads();
    // ---- (3) exp(lam) U, dq, dk, dg ----
    if (urole) {
      const float le = sLamE[cb * 16 + n16];
      float part = 0.f;  // rowsum(S_{n-1} * exp(lam) U_n), c = 16cb + n16
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        U[jb] *= le;  // exp(lam) U_n
        part += piece_dot(Sp[jb], U[jb]);
      }
      part = sum_over_g4(part);
      // dq^T[c][t] = sum_j S[c][j] dO[t][j] + ...;  dk^T[c][s] = sum_j (exp(lam)U)[c][j] V[s][j] + ...
      f32x4 aq[NTT], ak[NTT];
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) aq[tT] = ak[tT] = zero4();
#pragma unroll
      for (int j0 = 0; j0 < NJB; j0 += KU) {
        if constexpr (sizeof(E) == 2) {
          // merged, the lane's pieces of blocks j0 and j0 + 1 are the 8 adjacent columns
          // 16 j0 + pair_col(g4) + 0..7: the B fragment is one 16-byte read (two 8-byte reads
          // per fragment run at about a third of the rate)
          const bf16x8 xs = merge_pair(Sp[j0], Sp[j0 + 1]);
          const bf16x8 xu = merge_pair(to_bf16x4(U[j0]), to_bf16x4(U[j0 + 1]));
#pragma unroll
          for (int tT = 0; tT < NTT; ++tT) {
            const int off = (tT * 16 + n16) * LDV + 16 * j0 + pair_col(g4);
            aq[tT] = Mma<E>::mma(xs, *reinterpret_cast<const bf16x8*>(sdO + off), aq[tT]);
            ak[tT] = Mma<E>::mma(xu, *reinterpret_cast<const bf16x8*>(sV + off), ak[tT]);
          }
        } else {
          piece sp[1] = {Sp[j0]};
          f32x4 ue[1] = {U[j0]};
#pragma unroll
          for (int tT = 0; tT < NTT; ++tT) {
            const int t = tT * 16 + n16;
            aq[tT] = mma_regX_e<E, 1>(aq[tT], sp, sdO + t * LDV + j0 * 16);
            ak[tT] = mma_regX<1>(ak[tT], ue, sV + t * LDV + j0 * 16);
          }
        }
      }
      // the carry into this chunk from the later tokens, rowsum(S_n * U_n), formed as
      // rowsum(S_{n-1} * exp(lam) U_n) + sum_s k_s * dk_s|U_n (S_n = exp(lam) S_{n-1} + Ktil^T V): the
      // second term from the same U-part of dk^T that dg subtracts again below, so that where the
      // decay is strong the two cancel to float32 rounding, not to the stored state's
      f32x4 ku = zero4();
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) ku += load4(sK + (tT * 16 + n16) * LDK + cb * 16 + 4 * g4) * ak[tT];
      // + sum_s Kbar^T[c][s] dA[t][s] (s <= t);  + sum_t Qbar^T[c][t] dA^T[s][t] (t >= s): the Kbar^T and
      // Qbar^T fragments of this wave's rows are read once per k step for all row blocks
#pragma unroll
      for (int ks = 0; ks < C / KS; ++ks) {
        const typename Mma<E>::frag fk = frag_ld<E, true>(sK + cb * 16, LDK, ks * KS);
        const typename Mma<E>::frag fq = frag_ld<E, true>(sQ + cb * 16, LDQ, ks * KS);
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          if (ks * KS < (tT + 1) * 16) aq[tT] = Mma<E>::mma(fk, frag_ld<E, true>(sdAT + tT * 16, LDT, ks * KS), aq[tT]);
          if ((ks + 1) * KS > tT * 16) ak[tT] = Mma<E>::mma(fq, frag_ld<E, false>(sdAT + tT * 16 * LDT, LDT, ks * KS), ak[tT]);
        }
      }
      f32x4 xr[NTT];  // q dq - k dk at t = 16tT + n16, c = 16cb + 4g4 + i
      f32x4 dqt[2], dkt[2];
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) {
        const int t = tT * 16 + n16;
        const f32x4 q_ = aq[tT], k_ = ak[tT];
        const f32x4 lam4 = load4(sLam + t * LDQ + cb * 16 + 4 * g4);
        const f32x4 qb4 = load4(sQ + t * LDQ + cb * 16 + 4 * g4);
        const f32x4 kb4 = load4(sK + t * LDK + cb * 16 + 4 * g4);
        f32x4 rl;
#pragma unroll
        for (int i = 0; i < 4; ++i) rl[i] = __builtin_amdgcn_rcpf(lam4[i]);
        if constexpr (sizeof(E) == 2) {
          static_assert(NTT % 2 == 0, "token tiles pair up for bf16");
          dqt[tT & 1] = q_ * lam4;
          dkt[tT & 1] = k_ * rl;
          if (tT & 1) {
            // tiles tT - 1 and tT leave together, 16 bytes per lane: lane rows 0 and 2 store 8
            // channels of token 16(tT - 1) + n16, rows 1 and 3 those of token 16 tT + n16
            const long go = (t0 + 16 * (tT - 1 + (g4 & 1)) + n16) * DK + cb * 16 + 8 * (g4 >> 1);
            *reinterpret_cast<bf16x8*>(dq + go) = merge_pair(to_bf16x4(dqt[0]), to_bf16x4(dqt[1]));
            *reinterpret_cast<bf16x8*>(dk + go) = merge_pair(to_bf16x4(dkt[0]), to_bf16x4(dkt[1]));
          }
        } else {
          const long go = (t0 + t) * DK + cb * 16 + 4 * g4;
          store4(dq + go, q_ * lam4);
          store4(dk + go, k_ * rl);
        }
        xr[tT] = qb4 * q_ - kb4 * k_;
      }
      // dg[t][c] = sum_{t' >= t in the chunk} xr[t'][c] + carry[c]: suffix sums over the 16 tokens of
      // each row block (one DPP row: the lanes n16 of one g4), then over the later row blocks
      f32x4 later;
#pragma unroll
      for (int i = 0; i < 4; ++i) later[i] = __shfl(part, (l & ~15) | (4 * g4 + i)) + row_sum16(ku[i]);
#pragma unroll
      for (int tT = NTT - 1; tT >= 0; --tT) {
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float suf = seg_scan_rev_incl<16>(xr[tT][i]);
          d[i] = suf + later[i];
          later[i] += row_first(suf);
        }
        store4(dg + (t0 + tT * 16 + n16) * DK + cb * 16 + 4 * g4, d);
      }
    }
    __syncthreads();  // V and exp(b) are dead: the U staging area takes their place
    // ---- (4) dv = A^T dO + Kbar (exp(lam) U), half of d_v at a time; (5) U_{n-1} once the last half
    // of exp(lam) U is staged ----
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      if (urole) {
        if constexpr (sizeof(E) == 2) {  // pairs of 16-column blocks, 16 bytes per lane
#pragma unroll
          for (int jp = 0; jp < NJH / 2; ++jp)
            *reinterpret_cast<bf16x8*>(sU + (cb * 16 + n16) * LDU + jp * 32 + pair_col(g4)) =
                merge_pair(to_bf16x4(U[h * NJH + 2 * jp]), to_bf16x4(U[h * NJH + 2 * jp + 1]));
        } else {
#pragma unroll
          for (int jl = 0; jl < NJH; ++jl) {
            piece x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (E)U[h * NJH + jl][i];
            *reinterpret_cast<piece*>(sU + (cb * 16 + n16) * LDU + jl * 16 + 4 * g4) = x;
          }
        }
        if (h == NH - 1) {
          // (5) U_{n-1}^T[j][c] = exp(lam) U_n^T[j][c] + sum_t dO^T[j][t] Qbar^T[c][t]
#pragma unroll
          for (int ks = 0; ks < C / KS; ++ks) {
            const typename Mma<E>::frag fq = frag_ld<E, true>(sQ + cb * 16, LDQ, ks * KS);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
              U[jb] = Mma<E>::mma(frag_ld<E, true>(sdO + jb * 16, LDV, ks * KS), fq, U[jb]);
          }
        }
      }
      __syncthreads();
      // dv^T[j][s] = sum_t dO^T[j][t] A^T[s][t] + sum_c (exp(lam)U)^T[j][c] Kbar[s][c].  This wave takes
      // the row block sT = w % NTT and the column blocks jl = w / NTT, w / NTT + NW / NTT, ... (in
      // bf16, pairs of adjacent blocks, stored together); its A^T and Kbar fragments are read once
      // for all of them.
      {
        const int sT = w % NTT;
        typename Mma<E>::frag fa[C / KS], fkb[DK / KS];
#pragma unroll
        for (int ks = 0; ks < C / KS; ++ks)
          if ((ks + 1) * KS > sT * 16) fa[ks] = frag_ld<E, false>(sAT + sT * 16 * LDT, LDT, ks * KS);  // t >= s only
#pragma unroll
        for (int ks = 0; ks < DK / KS; ++ks) fkb[ks] = frag_ld<E, false>(sK + sT * 16 * LDK, LDK, ks * KS);
        auto dv_tile = [&](int jl) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < C / KS; ++ks)
            if ((ks + 1) * KS > sT * 16)
              acc = Mma<E>::mma(frag_ld<E, true>(sdO + h * DVH + jl * 16, LDV, ks * KS), fa[ks], acc);
#pragma unroll
          for (int ks = 0; ks < DK / KS; ++ks) acc = Mma<E>::mma(frag_ld<E, true>(sU + jl * 16, LDU, ks * KS), fkb[ks], acc);
          return acc;
        };
        E* const dvrow = dv + (t0 + sT * 16 + n16) * DV + h * DVH;
        if constexpr (sizeof(E) == 2) {
          static_assert(NJH % 2 == 0, "d_v blocks pair up for bf16");
          for (int jp = w / NTT; jp < NJH / 2; jp += NW / NTT) {
            const f32x4 x = dv_tile(2 * jp), y = dv_tile(2 * jp + 1);
            *reinterpret_cast<bf16x8*>(dvrow + jp * 32 + pair_col(g4)) = merge_pair(to_bf16x4(x), to_bf16x4(y));
          }
        } else {
          for (int jl = w / NTT; jl < NJH; jl += NW / NTT) store4(dvrow + jl * 16 + 4 * g4, dv_tile(jl));
        }
      }
      __syncthreads();
    }
  }
  // D = gradient w.r.t. the state entering the segment (from this segment's outputs); with
  // sub-segments the reverse scan over them gives it, with from_in the state-gradient pass
  if (urole && NS == 1 && !a.from_in) {
    float* dst = a.seg_dstate + (long)unit * SS;
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) store4(dst + (long)(cb * 16 + n16) * DV + jb * 16 + 4 * g4, U[jb]);
  }
  if (threadIdx.x == 0) a.flags[unit] = 0;
}

// State-gradient pass over sub-segments: from a zero gradient at the sub-segment's end, walking
// its chunks back, U_{n-1} = diag(exp(lam)) U_n + Qbar^T dO (Qbar = q exp(b)); the result is the
// gradient w.r.t. the state entering the sub-segment from its own outputs.  Every factor is
// exp(<= 0).  Wave w holds rows 16w .. of U, in bwd_kernel's lane layout.
// With a.reach the same gradient is summed from the other side: the chunks from the first one on,
// U += Qhat^T dO with Qhat_t = q_t exp(a_t), a_t the log-gates from the sub-segment's start
// through token t (b_t plus the earlier chunks' totals), and no decay of U.  Once every channel's
// running total is below kReachCut the later chunks' Qhat are exact zeros and the walk stops.
template <typename E, int C, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_state_kernel(BwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  typedef GateTile8<E, C, DK, NW * 64> GT;
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDV = lds_ld<E>(DV), LDQ = lds_ld<E>(DK);
  constexpr int NJB = DV / 16, NCB = DK / 16;
  constexpr int KS = Mma<E>::KSTEP;
  static_assert(NCB <= NW, "one 16-row block of U per wave");

  __shared__ __attribute__((aligned(16))) E sdO[C * LDV];  // dO   [t][j]
  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];   // Qbar [t][c]
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
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ dO = static_cast<const E*>(a.dO);
  const int NS = up.NS, sub = up.sub, seg = up.seg;
  const int L = a.T / a.P, Ls = L / NS, nchunks = Ls / C;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L + (long)sub * Ls;
  const int w = wave_id(), cb = w;
  const bool urole = cb < NCB;

  GT pgt;
  Vec8<E> pd[VPT];  // dO of the next chunk, requested with its gate tile
  auto prefetch = [&](int n, int tid) {
    pgt.load(a.g, q, nullptr, (tok0 + (long)n * C) * DK, tid);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pd[i].load(dO + (tok0 + (long)n * C + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
  };
  f32x4 U[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) U[jb] = zero4();
  // the summed log-gates of the chunks walked so far (every active lane, for its 8 channels)
  float ldsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // reach: walk from the first chunk, token t weighted by exp(log-gates from the start through t),
  // no decay of U; stop once every channel is past kReachCut
  const bool reach = a.reach && !a.list;

  prefetch(reach ? 0 : nchunks - 1, threadIdx.x);
  for (int it = 0; it < nchunks; ++it) {
    const int n = reach ? it : nchunks - 1 - it;
    const int tid = fresh_tid(), l = tid & 63, n16 = l & 15;
    {
      float b[GT::RI][8], lam[8];
      pgt.prefix(tid, sTot, b, lam);
      if (GT::active(tid)) {
        const int x = GT::group_of(tid);
        float before[8];  // log-gates before the chunk (reach), else 0
#pragma unroll
        for (int e = 0; e < 8; ++e) before[e] = reach ? ldsum[e] : 0.f;
#pragma unroll
        for (int r = 0; r < GT::RI; ++r) {
          float xq[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[e] = pgt.q[r].at(e) * __expf(b[r][e] + before[e]);
          store8(sQ + GT::row(tid, r) * LDQ + 8 * x, xq);
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
        if (NVP % NT == 0 || pc < NVP) pd[i].store(sdO + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < nchunks) prefetch(reach ? n + 1 : n - 1, tid);
    __syncthreads();
    if (urole) {
      // U^T[j][c] = exp(lam_c) U^T[j][c] + sum_t dO^T[j][t] Qbar^T[c][t]  (reach: no decay, the
      // weights are in Qbar)
      if (!reach) {
        const float le = sLamE[cb * 16 + n16];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) U[jb] *= le;
      }
#pragma unroll
      for (int ks = 0; ks < C / KS; ++ks) {
        const typename Mma<E>::frag fq = frag_ld<E, true>(sQ + cb * 16, LDQ, ks * KS);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) U[jb] = Mma<E>::mma(frag_ld<E, true>(sdO + jb * 16, LDV, ks * KS), fq, U[jb]);
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
  if (urole) {
    float* dst = up.st;
    const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) store4(dst + (long)(cb * 16 + n16) * DV + jb * 16 + 4 * g4, U[jb]);
  }
  const int tid = threadIdx.x;
  if (up.ld && GT::active(tid) && GT::set_of(tid) == 0 && (tid & 15) == 0)
    store8(up.ld + 8 * GT::group_of(tid), ldsum);
}

template <typename E, int C, int DK, int DV>
struct BwdLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.BH * a.P * a.S;
    hipLaunchKernelGGL((bwd_kernel<E, C, DK, DV, 8>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};

template <typename E, int C, int DK, int DV>
struct BwdStateLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.list ? 0 : a.BH * a.P * a.S;  // the units, or the re-split pieces' slots
    hipLaunchKernelGGL((bwd_state_kernel<E, C, DK, DV, 8>), dim3(a.list ? a.R : n_units), dim3(8 * 64), 0, s, a,
                       n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_bwd_state(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<BwdStateLauncher>(dtype, chunk, dk, dv);
}

launch_fn lookup_bwd(int dtype, int chunk, int dk, int dv) { return lookup_cdd<BwdLauncher>(dtype, chunk, dk, dv); }

}  // namespace gla
