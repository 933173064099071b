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
// ever runs over more than one chunk.  Two kernels walk every segment backwards: one over
// d_k slices (dq, dk, dg and the segment's local state gradient D), one over d_v slices (dv).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// ------------------------------------------------------------------------------------------
// dq, dk, dg, D: one workgroup per (unit, DKT-wide slice of d_k).  U^T[j][c] for the slice (all
// j) in accumulator registers; wave w owns the 16-row blocks cb = w, w+4, ...
// ------------------------------------------------------------------------------------------
template <typename E, int C, int DV, int DKT>
__global__ __launch_bounds__(kThreads) void bwd_dqk_kernel(BwdArgs a, int n_units) {
  constexpr int NTB = C / 8, NCB8 = DKT / 8, NKBLK = NTB * NCB8, NVB = NTB * (DV / 8);
  constexpr int LDV = DV + kPad, LDQ = DKT + kPad, LDT = C + kPad, LDL = DKT + 4;
  constexpr int NJB = DV / 16, NCB = DKT / 16, NTT = C / 16;
  constexpr int CPW = ceil_div(NCB, kWaves);
  constexpr int KS = Mma<E>::KSTEP;
  static_assert(NKBLK <= 128, "one 8x8 block of q and one of k per loader thread");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sdO[C * LDV];     // dO   [t][j]
  __shared__ __attribute__((aligned(16))) E sV[C * LDV];      // V    [s][j]
  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];      // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sK[C * LDQ];      // Kbar [s][c]
  __shared__ __attribute__((aligned(16))) E sdAT[C * LDT];    // dA^T [s][t], masked
  __shared__ __attribute__((aligned(16))) float sLam[C * LDL];  // exp(b) [t][c]
  __shared__ __attribute__((aligned(16))) float sX[C * LDL];    // q dq - k dk [t][c]
  __shared__ float sGtot[NTB * DKT];
  __shared__ float sXt[NTB * DKT];
  __shared__ float sLamE[DKT];
  __shared__ float sCarry[2][DKT];  // rowsum(S_n * U_n), by chunk parity

  const int Dk = a.Dk;
  const int NT = Dk / DKT;
  int unit, tile;
  xcd_map(blockIdx.x, NT, unit, tile);
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
  const long SS = (long)Dk * DV;  // one state
  const int c0 = tile * DKT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool krole = tid >= 128;
  const int bi = krole ? tid - 128 : tid;
  const bool has_blk = bi < NKBLK;
  const int tb = bi / NCB8, cb8 = bi - (bi / NCB8) * NCB8;

  f32x4 U[CPW][NJB];  // U[cc][jb][i] = U[c0 + 16cb + n16][16jb + 4g4 + i]
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc)
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) U[cc][jb] = zero4();
  if (tid < DKT) sCarry[(nchunks - 1) & 1][tid] = 0.f;  // nothing after the last chunk

  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    // global state before this chunk, same lane layout as U: Sp[cc][jb] = S[c][16jb + 4g4 + 0..3]
    piece Sp[CPW][NJB];
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * kWaves;
      const long roff = (long)(c0 + cb * 16 + n16) * DV + 4 * g4;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        if (cb >= NCB) {
          Sp[cc][jb] = piece{};
        } else if (n > 0) {
          Sp[cc][jb] = load_piece(cst + (chunk0 + n - 1) * SS + roff + jb * 16);
        } else {
          const f32x4 x = load4(a.seg_in + (long)unit * SS + roff + jb * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) Sp[cc][jb][i] = (E)x[i];
        }
      }
    }
    float gv[8][8], xv[8][8];
    if (has_blk) {
      load_blk<float>(gv, g + (t0 + tb * 8) * Dk + c0 + cb8 * 8, Dk);
      load_blk<E>(xv, (krole ? k : q) + (t0 + tb * 8) * Dk + c0 + cb8 * 8, Dk);
#pragma unroll
      for (int r = 1; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[r][e] += gv[r - 1][e];
      if (!krole)
#pragma unroll
        for (int e = 0; e < 8; ++e) sGtot[tb * DKT + cb8 * 8 + e] = gv[7][e];
    }
    for (int vb = tid; vb < NVB; vb += kThreads) {
      const int vtb = vb / (DV / 8), vjb = vb - (vb / (DV / 8)) * (DV / 8);
      float vv[8][8];
      load_blk<E>(vv, v + (t0 + vtb * 8) * DV + vjb * 8, DV);
      store_blk_rows<E>(sV + (vtb * 8) * LDV + vjb * 8, LDV, vv);
      load_blk<E>(vv, dO + (t0 + vtb * 8) * DV + vjb * 8, DV);
      store_blk_rows<E>(sdO + (vtb * 8) * LDV + vjb * 8, LDV, vv);
    }
    __syncthreads();
    if (has_blk) {
      float pre[8], tot[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { pre[e] = 0.f; tot[e] = 0.f; }
      for (int u = 0; u < NTB; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sGtot[u * DKT + cb8 * 8 + e];
          if (u < tb) pre[e] += s;
          tot[e] += s;
        }
      }
      if (!krole) {
        float lam[8][8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lam[r][e] = __expf(gv[r][e] + pre[e]);
            xv[r][e] *= lam[r][e];
          }
        store_blk_rows<E>(sQ + (tb * 8) * LDQ + cb8 * 8, LDQ, xv);
        store_blk_rows<float>(sLam + (tb * 8) * LDL + cb8 * 8, LDL, lam);
        if (tb == 0)
#pragma unroll
          for (int e = 0; e < 8; ++e) sLamE[cb8 * 8 + e] = __expf(tot[e]);
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[r][e] *= __expf(-(gv[r][e] + pre[e]));
        store_blk_rows<E>(sK + (tb * 8) * LDQ + cb8 * 8, LDQ, xv);
      }
    }
    __syncthreads();
    // dA[t][s] = dO[t] . V[s], stored as dA^T[s][t] for t >= s
    for (int idx = w; idx < NTT * NTT; idx += kWaves) {
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
    const int par = n & 1;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * kWaves;
      if (cb < NCB) {
        const float le = sLamE[cb * 16 + n16];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) U[cc][jb] *= le;  // exp(lam) U_n
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const int t = tT * 16 + n16;  // the token of this lane's column (t for dq, s for dk)
          // dq^T[c][t] = sum_j S[c][j] dO[t][j] + sum_s Kbar^T[c][s] dA[t][s]
          f32x4 aq = mma_regX_e<E, NJB>(zero4(), Sp[cc], sdO + t * LDV);
          const int ke = round_up((tT + 1) * 16, KS) < C ? round_up((tT + 1) * 16, KS) : C;
          aq = mma<E, true, true>(aq, sK + cb * 16, LDQ, sdAT + tT * 16, LDT, 0, ke);
          // dk^T[c][s] = sum_t Qbar^T[c][t] dA^T[s][t] + sum_j (exp(lam)U)[c][j] V[s][j]
          f32x4 ak = mma<E, true, false>(zero4(), sQ + cb * 16, LDQ, sdAT + tT * 16 * LDT, LDT,
                                         (tT * 16 / KS) * KS, C);
          ak = mma_regX<E, NJB>(ak, U[cc], sV + t * LDV);
          const f32x4 lam4 = load4(sLam + t * LDL + cb * 16 + 4 * g4);
          const f32x4 qb4 = load4(sQ + t * LDQ + cb * 16 + 4 * g4);
          const f32x4 kb4 = load4(sK + t * LDQ + cb * 16 + 4 * g4);
          const long go = (t0 + t) * Dk + c0 + cb * 16 + 4 * g4;
          store4(dq + go, aq * lam4);
          store4(dk + go, ak / lam4);
          store4(sX + t * LDL + cb * 16 + 4 * g4, qb4 * aq - kb4 * ak);  // q dq - k dk
        }
        // U_{n-1}: U^T[j][c] += sum_t dO^T[j][t] Qbar^T[c][t]
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
          U[cc][jb] = mma<E, true, true>(U[cc][jb], sdO + jb * 16, LDV, sQ + cb * 16, LDQ, 0, C);
        // carry into chunk n-1: rowsum(S_{n-1} * U_{n-1})
        float part = 0.f;
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) part += piece_dot(Sp[cc][jb], U[cc][jb]);
        part = sum_over_g4(part);
        if (g4 == 0) sCarry[par ^ 1][cb * 16 + n16] = part;
      }
    }
    __syncthreads();
    // dg: in-chunk reverse running sum of q dq - k dk plus the exact carry
    float xs[8][8];
    if (krole && has_blk) {
#pragma unroll
      for (int r = 0; r < 8; ++r) load8(sX + (tb * 8 + r) * LDL + cb8 * 8, xs[r]);
#pragma unroll
      for (int r = 6; r >= 0; --r)
#pragma unroll
        for (int e = 0; e < 8; ++e) xs[r][e] += xs[r + 1][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) sXt[tb * DKT + cb8 * 8 + e] = xs[0][e];
    }
    __syncthreads();
    if (krole && has_blk) {
      float suf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) suf[e] = sCarry[par][cb8 * 8 + e];
      for (int u = NTB - 1; u > tb; --u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) suf[e] += sXt[u * DKT + cb8 * 8 + e];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float outv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) outv[e] = xs[r][e] + suf[e];
        store8(dg + (t0 + tb * 8 + r) * Dk + c0 + cb8 * 8, outv);
      }
    }
    __syncthreads();
  }
  // D = gradient w.r.t. the state entering the segment (from this segment's outputs)
  float* dst = a.seg_dstate + (long)unit * SS;
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int cb = w + cc * kWaves;
    if (cb < NCB)
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) store4(dst + (long)(c0 + cb * 16 + n16) * DV + jb * 16 + 4 * g4, U[cc][jb]);
  }
}

// ------------------------------------------------------------------------------------------
// dv: one workgroup per (unit, DVT-wide slice of d_v), walking backwards.  U[c][j] for the
// slice, all c, starts at zero.
// ------------------------------------------------------------------------------------------
template <typename E, int C, int DK, int DVT>
__global__ __launch_bounds__(kThreads) void bwd_dv_kernel(BwdArgs a, int n_units) {
  constexpr int NTB = C / 8, NCB8 = DK / 8, NQB = NTB * NCB8, NVB = NTB * (DVT / 8);
  constexpr int LDQ = DK + kPad, LDV = DVT + kPad, LDT = C + kPad;
  constexpr int NJB = DVT / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, kWaves);
  constexpr int KS = Mma<E>::KSTEP;
  static_assert(NQB <= 128, "one 8x8 block of q and one of k per loader thread");

  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];    // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sK[C * LDQ];    // Kbar [s][c]
  __shared__ __attribute__((aligned(16))) E sdO[C * LDV];   // dO   [t][j]
  __shared__ __attribute__((aligned(16))) E sAT[C * LDT];   // A^T  [s][t], masked
  __shared__ float sGtot[NTB * DK];
  __shared__ float sLamE[DK];

  const int Dv = a.Dv;
  const int NT = Dv / DVT;
  int unit, tile;
  xcd_map(blockIdx.x, NT, unit, tile);
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ dO = static_cast<const E*>(a.dO);
  const float* __restrict__ g = a.g;
  E* __restrict__ dv = static_cast<E*>(a.dv);
  const int L = a.T / a.P;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const int j0 = tile * DVT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool krole = tid >= 128;
  const int bi = krole ? tid - 128 : tid;
  const bool has_blk = bi < NQB;
  const int tb = bi / NCB8, cb8 = bi - (bi / NCB8) * NCB8;

  f32x4 U[JPW][NKB];  // U[jj][kb][i] = U[16kb + 4g4 + i][j0 + 16jb + n16]
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) U[jj][kb] = zero4();

  const int nchunks = L / C;
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    float gv[8][8], xv[8][8];
    if (has_blk) {
      load_blk<float>(gv, g + (t0 + tb * 8) * DK + cb8 * 8, DK);
      load_blk<E>(xv, (krole ? k : q) + (t0 + tb * 8) * DK + cb8 * 8, DK);
#pragma unroll
      for (int r = 1; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[r][e] += gv[r - 1][e];
      if (!krole)
#pragma unroll
        for (int e = 0; e < 8; ++e) sGtot[tb * DK + cb8 * 8 + e] = gv[7][e];
    }
    for (int vb = tid; vb < NVB; vb += kThreads) {
      const int vtb = vb / (DVT / 8), vjb = vb - (vb / (DVT / 8)) * (DVT / 8);
      float vv[8][8];
      load_blk<E>(vv, dO + (t0 + vtb * 8) * Dv + j0 + vjb * 8, Dv);
      store_blk_rows<E>(sdO + (vtb * 8) * LDV + vjb * 8, LDV, vv);
    }
    __syncthreads();
    if (has_blk) {
      float pre[8], tot[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { pre[e] = 0.f; tot[e] = 0.f; }
      for (int u = 0; u < NTB; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sGtot[u * DK + cb8 * 8 + e];
          if (u < tb) pre[e] += s;
          tot[e] += s;
        }
      }
      if (!krole) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[r][e] *= __expf(gv[r][e] + pre[e]);
        store_blk_rows<E>(sQ + (tb * 8) * LDQ + cb8 * 8, LDQ, xv);
        if (tb == 0)
#pragma unroll
          for (int e = 0; e < 8; ++e) sLamE[cb8 * 8 + e] = __expf(tot[e]);
      } else {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) xv[r][e] *= __expf(-(gv[r][e] + pre[e]));
        store_blk_rows<E>(sK + (tb * 8) * LDQ + cb8 * 8, LDQ, xv);
      }
    }
    __syncthreads();
    // A[t][s] = Qbar[t] . Kbar[s], stored transposed as A^T[s][t] for t >= s
    for (int idx = w; idx < NTT * NTT; idx += kWaves) {
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
      const int jb = w + jj * kWaves;
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
          store4(dv + (t0 + sT * 16 + n16) * Dv + j0 + jb * 16 + 4 * g4, acc);
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

template <typename E, int C, int DV, int DKT>
struct BwdDqkLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.BH * a.P;
    const dim3 grid(round_up(n_units, 8) * (a.Dk / DKT));
    hipLaunchKernelGGL((bwd_dqk_kernel<E, C, DV, DKT>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};
template <typename E, int C, int DK, int DVT>
struct BwdDvLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const BwdArgs& a = *static_cast<const BwdArgs*>(pa);
    const int n_units = a.BH * a.P;
    const dim3 grid(round_up(n_units, 8) * (a.Dv / DVT));
    hipLaunchKernelGGL((bwd_dv_kernel<E, C, DK, DVT>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_bwd_dqk(int dtype, int chunk, int dk, int dv) {
  return lookup3<BwdDqkLauncher, Bf16Dv, F32Dv>(dtype, chunk, dv, tile_of(dk));
}
launch_fn lookup_bwd_dv(int dtype, int chunk, int dk, int dv) {
  return lookup3<BwdDvLauncher, Bf16Dk, F32Dk>(dtype, chunk, dk, tile_of(dv));
}

}  // namespace gla
