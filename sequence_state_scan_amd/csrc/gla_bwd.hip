// Backward kernels of the chunkwise form, per segment, given the GLOBAL state after every chunk
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
// ever runs over more than one chunk.  Two kernels walk every segment backwards, one workgroup
// of NW waves per segment each: one keeps U^T (all of d_v, all of d_k) for dq, dk, dg and the
// segment's local state gradient D; the other keeps U for dv.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// ------------------------------------------------------------------------------------------
// dq, dk, dg, D: one workgroup per unit; wave w owns the 16-row blocks cb = w, w+NW, ... of
// U^T[j][c] (all j) and of the chunk state it reads for dq.
// ------------------------------------------------------------------------------------------
template <typename E, int C, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dqk_kernel(BwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  constexpr int NTG = C / 4, NCG = DK / 8, NI = NTG * NCG, RT = NT / 2;
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDV = DV + kPad, LDQ = DK + kPad, LDT = C + kPad, LDX = DK + 4;
  constexpr int NJB = DV / 16, NCB = DK / 16, NTT = C / 16;
  constexpr int CPW = ceil_div(NCB, NW);
  constexpr int KS = Mma<E>::KSTEP;
  constexpr int KU = sizeof(E) == 2 ? 2 : 1;  // 16-wide d_v blocks per k-step of the MFMA
  constexpr int RAWB = (C * LDV * (int)sizeof(E) > C * LDX * 4) ? C * LDV * (int)sizeof(E) : C * LDX * 4;
  static_assert(NI <= RT, "one 4x8 item of q (and one of k) per loader thread");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sdO[C * LDV];          // dO   [t][j]
  __shared__ __attribute__((aligned(16))) unsigned char sRaw[RAWB];  // V [s][j], then x [t][c] (f32)
  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];           // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sK[C * LDQ];           // Kbar [s][c]
  __shared__ __attribute__((aligned(16))) E sLam[C * LDQ];         // exp(b) [t][c]
  __shared__ __attribute__((aligned(16))) E sdAT[C * LDT];         // dA^T [s][t], masked
  __shared__ float sLamE[DK];
  __shared__ float sCarry[2][DK];  // rowsum(S_n * U_n), by chunk parity
  E* const sV = reinterpret_cast<E*>(sRaw);
  float* const sX = reinterpret_cast<float*>(sRaw);

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
  float* __restrict__ dg = a.dg;
  const int L = a.T / a.P;
  const int nchunks = L / C;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const long chunk0 = (long)unit * nchunks;
  const long SS = (long)DK * DV;  // one state
  const int w = wave_id();
  typedef LoaderRole<RT, NTG, NI> Role;

  Rows4x8<float> pg;
  Rows4x8<E> px;
  auto prefetch = [&](int n, int tid) {
    const Role r(tid);
    const long t0 = tok0 + (long)n * C;
    if (r.has_item) {
      pg.load(g + (t0 + r.tg * 4) * DK + r.cg * 8, DK);
      px.load((r.krole ? k : q) + (t0 + r.tg * 4) * DK + r.cg * 8, DK);
    }
  };

  f32x4 U[CPW][NJB];  // U[cc][jb][i] = U[16cb + n16][16jb + 4g4 + i]
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) U[cc][jb] = zero4();
  if (threadIdx.x < DK) sCarry[(nchunks - 1) & 1][threadIdx.x] = 0.f;  // nothing after the last chunk

  prefetch(nchunks - 1, threadIdx.x);
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    const int tid = fresh_tid(), l = tid & 63, n16 = l & 15, g4 = l >> 4;
    const Role role(tid);
    const bool krole = role.krole, has_item = role.has_item;
    const int tg = role.tg, cg = role.cg;
    // this chunk's V and dO, and the global state before it (same lane layout as U)
    Vec8<E> pv[VPT], pd[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) {
        const long off = (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8;
        pv[i].load(v + off);
        pd[i].load(dO + off);
      }
    }
    // ---- (1) gate prefix sums, Qbar, Kbar, exp(b); V, dO -> LDS ----
    {
      float b[4][8], lam[8];
      chunk_gate_prefix<NTG>(pg, has_item, b, lam);
      if (has_item) {
        if (!krole) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[8], e8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              e8[e] = __expf(b[r][e]);
              x[e] = px.at(r, e) * e8[e];
            }
            store8(sQ + (tg * 4 + r) * LDQ + cg * 8, x);
            store8(sLam + (tg * 4 + r) * LDQ + cg * 8, e8);
          }
          if (tg == 0)
#pragma unroll
            for (int e = 0; e < 8; ++e) sLamE[cg * 8 + e] = __expf(lam[e]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = px.at(r, e) * __expf(-b[r][e]);
            store8(sK + (tg * 4 + r) * LDQ + cg * 8, x);
          }
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
    piece Sp[CPW][NJB];
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * NW;
      const long roff = (long)(cb * 16 + n16) * DV + 4 * g4;
      if (cb >= NCB) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) Sp[cc][jb] = piece{};
      } else if (n > 0) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) Sp[cc][jb] = load_piece(cst + (chunk0 + n - 1) * SS + roff + jb * 16);
      } else {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const f32x4 x = load4(a.seg_in + (long)unit * SS + roff + jb * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) Sp[cc][jb][i] = (E)x[i];
        }
      }
    }
    __syncthreads();
    // ---- (2) dA[t][s] = dO[t] . V[s], stored as dA^T[s][t] for t >= s ----
    for (int idx = w; idx < NTT * NTT; idx += NW) {
      const int tT = idx / NTT, sT = idx - (idx / NTT) * NTT;
      f32x4 acc = zero4();
      if (sT <= tT) acc = mma<E, false, false>(acc, sdO + tT * 16 * LDV, LDV, sV + sT * 16 * LDV, LDV, 0, DV);
      const int s = sT * 16 + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tT * 16 + 4 * g4 + i < s) acc[i] = 0.f;
      store4(sdAT + s * LDT + tT * 16 + 4 * g4, acc);
    }
    __syncthreads();
    // ---- (3) dq, dk, the U update and the next carry ----
    // The d_v sum of dq (over the chunk state) and of dk (over exp(lam) U) runs in KU-block steps
    // so that only one step's worth of the chunk state is live at a time.
    const int par = n & 1;
    f32x4 xr[CPW][NTT];  // q dq - k dk for this wave's rows, accumulator layout
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * NW;
      if (cb < NCB) {
        const float le = sLamE[cb * 16 + n16];
        f32x4 aq[NTT], ak[NTT];
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) aq[tT] = ak[tT] = zero4();
        float part = 0.f;
#pragma unroll
        for (int j0 = 0; j0 < NJB; j0 += KU) {
          piece sp[KU];
          f32x4 ue[KU];
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            sp[u] = Sp[cc][j0 + u];
            ue[u] = U[cc][j0 + u] * le;  // exp(lam) U_n
          }
#pragma unroll
          for (int tT = 0; tT < NTT; ++tT) {
            const int t = tT * 16 + n16;
            // dq^T[c][t] += sum_j S[c][j] dO[t][j];  dk^T[c][s] += sum_j (exp(lam)U)[c][j] V[s][j]
            aq[tT] = mma_regX_e<E, KU>(aq[tT], sp, sdO + t * LDV + j0 * 16);
            ak[tT] = mma_regX<E, KU>(ak[tT], ue, sV + t * LDV + j0 * 16);
          }
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            // U_{n-1}: U^T[j][c] = exp(lam) U_n^T[j][c] + sum_t dO^T[j][t] Qbar^T[c][t]
            U[cc][j0 + u] = mma<E, true, true>(ue[u], sdO + (j0 + u) * 16, LDV, sQ + cb * 16, LDQ, 0, C);
            part += piece_dot(sp[u], U[cc][j0 + u]);  // carry into chunk n-1: rowsum(S_{n-1} * U_{n-1})
          }
        }
        part = sum_over_g4(part);
        if (g4 == 0) sCarry[par ^ 1][cb * 16 + n16] = part;
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const int t = tT * 16 + n16;  // the token of this lane's column (t for dq, s for dk)
          // dq^T[c][t] += sum_s Kbar^T[c][s] dA[t][s];  dk^T[c][s] += sum_t Qbar^T[c][t] dA^T[s][t]
          const int ke = round_up((tT + 1) * 16, KS) < C ? round_up((tT + 1) * 16, KS) : C;
          const f32x4 q_ = mma<E, true, true>(aq[tT], sK + cb * 16, LDQ, sdAT + tT * 16, LDT, 0, ke);
          const f32x4 k_ = mma<E, true, false>(ak[tT], sQ + cb * 16, LDQ, sdAT + tT * 16 * LDT, LDT,
                                               (tT * 16 / KS) * KS, C);
          const f32x4 lam4 = load4(sLam + t * LDQ + cb * 16 + 4 * g4);
          const f32x4 qb4 = load4(sQ + t * LDQ + cb * 16 + 4 * g4);
          const f32x4 kb4 = load4(sK + t * LDQ + cb * 16 + 4 * g4);
          const long go = (t0 + t) * DK + cb * 16 + 4 * g4;
          store4(dq + go, q_ * lam4);
          store4(dk + go, k_ / lam4);
          xr[cc][tT] = qb4 * q_ - kb4 * k_;  // q dq - k dk
        }
      }
    }
    __syncthreads();  // V is dead: its space takes x
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * NW;
      if (cb < NCB)
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) store4(sX + (tT * 16 + n16) * LDX + cb * 16 + 4 * g4, xr[cc][tT]);
    }
    __syncthreads();
    // ---- (4) dg: in-chunk reverse running sum of q dq - k dk plus the exact carry ----
    if (!krole) {
      float xs[4][8], suf[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (has_item) load8(sX + (tg * 4 + r) * LDX + cg * 8, xs[r]);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[r][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float run = 0.f;
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          run += xs[r][e];
          xs[r][e] = run;
        }
        const float incl = seg_scan_rev_incl<NTG>(run);
        suf[e] = seg_next<NTG>(incl) + (has_item ? sCarry[par][cg * 8 + e] : 0.f);
      }
      if (has_item)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float outv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) outv[e] = xs[r][e] + suf[e];
          store8(dg + (t0 + tg * 4 + r) * DK + cg * 8, outv);
        }
    }
    __syncthreads();
  }
  // D = gradient w.r.t. the state entering the segment (from this segment's outputs)
  float* dst = a.seg_dstate + (long)unit * SS;
  const int n16 = lane_id() & 15, g4 = lane_id() >> 4;
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int cb = w + cc * NW;
    if (cb < NCB)
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) store4(dst + (long)(cb * 16 + n16) * DV + jb * 16 + 4 * g4, U[cc][jb]);
  }
}

// ------------------------------------------------------------------------------------------
// dv: one workgroup per unit; wave w owns the 16-column blocks jb = w, w+NW, ... of U[c][j]
// (all c).
// ------------------------------------------------------------------------------------------
template <typename E, int C, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dv_kernel(BwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  constexpr int NTG = C / 4, NCG = DK / 8, NI = NTG * NCG, RT = NT / 2;
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDQ = DK + kPad, LDV = DV + kPad, LDT = C + kPad;
  constexpr int NJB = DV / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, NW);
  constexpr int KS = Mma<E>::KSTEP;
  static_assert(NI <= RT, "one 4x8 item of q (and one of k) per loader thread");

  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];    // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sK[C * LDQ];    // Kbar [s][c]
  __shared__ __attribute__((aligned(16))) E sdO[C * LDV];   // dO   [t][j]
  __shared__ __attribute__((aligned(16))) E sAT[C * LDT];   // A^T  [s][t], masked
  __shared__ float sLamE[DK];

  const int unit = blockIdx.x;
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ dO = static_cast<const E*>(a.dO);
  const float* __restrict__ g = a.g;
  E* __restrict__ dv = static_cast<E*>(a.dv);
  const int L = a.T / a.P;
  const int nchunks = L / C;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool krole = tid >= RT;
  const int rt = krole ? tid - RT : tid;
  const bool has_item = rt < NI;
  const int tg = rt % NTG, cg = rt / NTG;
  const E* __restrict__ xsrc = krole ? k : q;

  Rows4x8<float> pg;
  Rows4x8<E> px;
  Vec8<E> pd[VPT];
  auto prefetch = [&](int n) {
    const long t0 = tok0 + (long)n * C;
    if (has_item) {
      pg.load(g + (t0 + tg * 4) * DK + cg * 8, DK);
      px.load(xsrc + (t0 + tg * 4) * DK + cg * 8, DK);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pd[i].load(dO + (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
  };

  f32x4 U[JPW][NKB];  // U[jj][kb][i] = U[16kb + 4g4 + i][16jb + n16]
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) U[jj][kb] = zero4();

  prefetch(nchunks - 1);
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    {
      float b[4][8], lam[8];
      chunk_gate_prefix<NTG>(pg, has_item, b, lam);
      if (has_item) {
        if (!krole) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = px.at(r, e) * __expf(b[r][e]);
            store8(sQ + (tg * 4 + r) * LDQ + cg * 8, x);
          }
          if (tg == 0)
#pragma unroll
            for (int e = 0; e < 8; ++e) sLamE[cg * 8 + e] = __expf(lam[e]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = px.at(r, e) * __expf(-b[r][e]);
            store8(sK + (tg * 4 + r) * LDQ + cg * 8, x);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int pc = tid + NT * i;
        if (NVP % NT == 0 || pc < NVP) pd[i].store(sdO + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (n > 0) prefetch(n - 1);
    __syncthreads();
    // A[t][s] = Qbar[t] . Kbar[s], stored transposed as A^T[s][t] for t >= s
    for (int idx = w; idx < NTT * NTT; idx += NW) {
      const int tT = idx / NTT, sT = idx - (idx / NTT) * NTT;
      f32x4 acc = zero4();
      if (sT <= tT) acc = mma<E, false, false>(acc, sQ + tT * 16 * LDQ, LDQ, sK + sT * 16 * LDQ, LDQ, 0, DK);
      const int s = sT * 16 + n16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tT * 16 + 4 * g4 + i < s) acc[i] = 0.f;
      store4(sAT + s * LDT + tT * 16 + 4 * g4, acc);
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w + jj * NW;
      if (jb < NJB) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) U[jj][kb][i] *= sLamE[kb * 16 + 4 * g4 + i];  // exp(lam) U
        // dv^T[j][s] = sum_t dO^T[j][t] A^T[s][t] + sum_c (exp(lam)U)^T[j][c] Kbar[s][c]
#pragma unroll
        for (int sT = 0; sT < NTT; ++sT) {
          f32x4 acc = mma<E, true, false>(zero4(), sdO + jb * 16, LDV, sAT + sT * 16 * LDT, LDT,
                                          (sT * 16 / KS) * KS, C);
          acc = mma_regX<E, NKB>(acc, U[jj], sK + (sT * 16 + n16) * LDQ);
          store4(dv + (t0 + sT * 16 + n16) * DV + jb * 16 + 4 * g4, acc);
        }
        // U[c][j] += sum_t Qbar^T[c][t] dO^T[j][t]
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          U[jj][kb] = mma<E, true, true>(U[jj][kb], sQ + kb * 16, LDQ, sdO + jb * 16, LDV, 0, C);
      }
    }
    __syncthreads();
  }
}

template <typename E, int C, int DK, int DV>
struct BwdDqkLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.BH * a.P;
    hipLaunchKernelGGL((bwd_dqk_kernel<E, C, DK, DV, 8>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};
template <typename E, int C, int DK, int DV>
struct BwdDvLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.BH * a.P;
    hipLaunchKernelGGL((bwd_dv_kernel<E, C, DK, DV, 8>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_bwd_dqk(int dtype, int chunk, int dk, int dv) { return lookup_cdd<BwdDqkLauncher>(dtype, chunk, dk, dv); }
launch_fn lookup_bwd_dv(int dtype, int chunk, int dk, int dv) { return lookup_cdd<BwdDvLauncher>(dtype, chunk, dk, dv); }

}  // namespace gla
