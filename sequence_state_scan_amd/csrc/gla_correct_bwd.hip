// Backward correction: add the later segments' state gradient G_p to every segment's local
// dk, dv and dg.  For t in segment p, with r_t = sum of g over the tokens after t up to the
// segment's end:
//   dk[t] += exp(r_t) * (G_p v_t)
//   dv[t] += G_p^T (exp(r_t) * k_t)
//   dg[t] += exp(g_t + r_t) * rowsum(S_{t-1} * G_p)        (the direct form of dg, S global)
// In chunk n the last line is E_n * R_n + sum_{s < t in chunk n} k_s * (exp(r_s) G_p v_s), with
// R_n = rowsum(S_{n-1} * G_p) from the stored global state before the chunk and E_n = exp(sum of
// g from the chunk's first token to the segment's end).  Every term carries a decay to the
// segment's end, so the loops walk each segment from its end; with g <= 0 the decays only shrink
// going back, and once a whole chunk has exp(r_t) == 0.0f nothing before it changes.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// dk and dg: one workgroup per (unit, DKT-wide slice of d_k).  G[c][:] for the slice sits in
// registers (wave w owns the 16-row blocks cb = w, w+4, ...) and feeds the MFMA A operand.
template <typename E, int C, int DV, int DKT>
__global__ __launch_bounds__(kThreads) void correct_bwd_dk_kernel(CorrArgs a, int n_units) {
  constexpr int NTB = C / 8, NCB8 = DKT / 8, NKBLK = NTB * NCB8, NVB = NTB * (DV / 8);
  constexpr int LDV = DV + kPad, LDL = DKT + 4;
  constexpr int NJB = DV / 16, NCB = DKT / 16, NTT = C / 16;
  constexpr int CPW = ceil_div(NCB, kWaves);
  static_assert(NKBLK <= kThreads, "one 8x8 block per loader thread");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sV[C * LDV];      // V [t][j]
  __shared__ __attribute__((aligned(16))) float sE[C * LDL];  // exp(r_t) [t][c]
  __shared__ __attribute__((aligned(16))) float sKD[C * LDL]; // k * delta-dk [t][c]
  __shared__ float sGtot[NTB * DKT];
  __shared__ float sXt[NTB * DKT];
  __shared__ float sEn[DKT];  // E_n
  __shared__ float sR[DKT];   // R_n

  const int Dk = a.Dk;
  const int NT = Dk / DKT;
  int unit, tile;
  xcd_map(blockIdx.x, NT, unit, tile);
  if (unit >= n_units) return;
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const E* __restrict__ cst = static_cast<const E*>(a.chunk_states);
  const float* __restrict__ g = a.g;
  E* __restrict__ dk = static_cast<E*>(a.dk);
  float* __restrict__ dg = a.dg;
  const int L = a.T / a.P;
  const int nchunks = L / C;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const long chunk0 = (long)unit * nchunks;
  const long SS = (long)Dk * DV;
  const int c0 = tile * DKT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool has_blk = tid < NKBLK;
  const int tb = tid / NCB8, cb8 = tid - (tid / NCB8) * NCB8;

  // G slice: R[cc][jb][i] = G[c0 + 16cb + n16][16jb + 4g4 + i]
  const float* gp = a.seg_grad + (long)unit * SS;
  f32x4 R[CPW][NJB];
  int nonzero = 0;
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int cb = w + cc * kWaves;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      R[cc][jb] = cb < NCB ? load4(gp + (long)(c0 + cb * 16 + n16) * DV + jb * 16 + 4 * g4) : zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) nonzero |= R[cc][jb][i] != 0.f;
    }
  }
  if (!__syncthreads_or(nonzero)) return;  // G_p == 0: nothing to add

  float gcarry[8];  // sum of g from the segment's end back to the current chunk (loader threads)
#pragma unroll
  for (int e = 0; e < 8; ++e) gcarry[e] = 0.f;
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    // global state before this chunk, in G's lane layout
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
    float gv[8][8];
    int live = 0;
    if (has_blk) {
      load_blk<float>(gv, g + (t0 + tb * 8) * Dk + c0 + cb8 * 8, Dk);
      float tot[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        tot[e] = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) tot[e] += gv[r][e];
        sGtot[tb * DKT + cb8 * 8 + e] = tot[e];
      }
    }
    for (int vb = tid; vb < NVB; vb += kThreads) {
      const int vtb = vb / (DV / 8), vjb = vb - (vb / (DV / 8)) * (DV / 8);
      float vv[8][8];
      load_blk<E>(vv, v + (t0 + vtb * 8) * DV + vjb * 8, DV);
      store_blk_rows<E>(sV + (vtb * 8) * LDV + vjb * 8, LDV, vv);
    }
    __syncthreads();
    if (has_blk) {
      float run[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = gcarry[e];
      for (int u = NTB - 1; u >= 0; --u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sGtot[u * DKT + cb8 * 8 + e];
          if (u > tb) run[e] += s;
          gcarry[e] += s;
        }
      }
      // exclusive: tokens strictly after t (within the segment)
#pragma unroll
      for (int r = 7; r >= 0; --r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ex = __expf(run[e]);
          run[e] += gv[r][e];
          gv[r][e] = ex;
          live |= ex != 0.f;
        }
      store_blk_rows<float>(sE + (tb * 8) * LDL + cb8 * 8, LDL, gv);
      if (tb == 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) sEn[cb8 * 8 + e] = __expf(gcarry[e]);
    }
    if (!__syncthreads_or(live)) break;
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * kWaves;
      if (cb < NCB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const int t = tT * 16 + n16;
          f32x4 acc = mma_regX<E, NJB>(zero4(), R[cc], sV + t * LDV);  // (G v_t)[c]
          acc *= load4(sE + t * LDL + cb * 16 + 4 * g4);
          E* dkp = dk + (t0 + t) * Dk + c0 + cb * 16 + 4 * g4;
          const f32x4 kk = load4(k + (t0 + t) * Dk + c0 + cb * 16 + 4 * g4);
          store4(dkp, load4(dkp) + acc);
          store4(sKD + t * LDL + cb * 16 + 4 * g4, kk * acc);
        }
        float part = 0.f;  // R_n = rowsum(S_{n-1} * G)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) part += piece_dot(Sp[cc][jb], R[cc][jb]);
        part = sum_over_g4(part);
        if (g4 == 0) sR[cb * 16 + n16] = part;
      }
    }
    __syncthreads();
    float xs[8][8];
    if (has_blk) {
#pragma unroll
      for (int r = 0; r < 8; ++r) load8(sKD + (tb * 8 + r) * LDL + cb8 * 8, xs[r]);
      // exclusive prefix over the block's tokens
      float run[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = 0.f;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = xs[r][e];
          xs[r][e] = run[e];
          run[e] += x;
        }
#pragma unroll
      for (int e = 0; e < 8; ++e) sXt[tb * DKT + cb8 * 8 + e] = run[e];
    }
    __syncthreads();
    if (has_blk) {
      float base[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) base[e] = sEn[cb8 * 8 + e] * sR[cb8 * 8 + e];
      for (int u = 0; u < tb; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) base[e] += sXt[u * DKT + cb8 * 8 + e];
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        float* dgp = dg + (t0 + tb * 8 + r) * Dk + c0 + cb8 * 8;
        float cur[8];
        load8(dgp, cur);
#pragma unroll
        for (int e = 0; e < 8; ++e) cur[e] += base[e] + xs[r][e];
        store8(dgp, cur);
      }
    }
    __syncthreads();
  }
}

// dv: one workgroup per (unit, DVT-wide slice of d_v).  G^T[j][:] for the slice in registers.
template <typename E, int C, int DK, int DVT>
__global__ __launch_bounds__(kThreads) void correct_bwd_dv_kernel(CorrArgs a, int n_units) {
  constexpr int NTB = C / 8, NCB8 = DK / 8, NQB = NTB * NCB8;
  constexpr int LDQ = DK + kPad;
  constexpr int NJB = DVT / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, kWaves);
  static_assert(NQB <= kThreads, "one 8x8 block per loader thread");

  __shared__ __attribute__((aligned(16))) E sEK[C * LDQ];  // e_t * k_t [t][c]
  __shared__ float sGtot[NTB * DK];

  const int Dv = a.Dv;
  const int NT = Dv / DVT;
  int unit, tile;
  xcd_map(blockIdx.x, NT, unit, tile);
  if (unit >= n_units) return;
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const float* __restrict__ g = a.g;
  E* __restrict__ dv = static_cast<E*>(a.dv);
  const int L = a.T / a.P;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const int j0 = tile * DVT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool has_blk = tid < NQB;
  const int tb = tid / NCB8, cb8 = tid - (tid / NCB8) * NCB8;

  // G^T slice: R[jj][kb][i] = G[16kb + 4g4 + i][j0 + 16jb + n16]
  const float* gp = a.seg_grad + (long)unit * DK * Dv;
  f32x4 R[JPW][NKB];
  int nonzero = 0;
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int jb = w + jj * kWaves;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        R[jj][kb][i] = jb < NJB ? gp[(long)(kb * 16 + 4 * g4 + i) * Dv + j0 + jb * 16 + n16] : 0.f;
        nonzero |= R[jj][kb][i] != 0.f;
      }
  }
  if (!__syncthreads_or(nonzero)) return;

  float gcarry[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gcarry[e] = 0.f;
  const int nchunks = L / C;
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    float gv[8][8], kv[8][8];
    int live = 0;
    if (has_blk) {
      load_blk<float>(gv, g + (t0 + tb * 8) * DK + cb8 * 8, DK);
      load_blk<E>(kv, k + (t0 + tb * 8) * DK + cb8 * 8, DK);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float tot = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) tot += gv[r][e];
        sGtot[tb * DK + cb8 * 8 + e] = tot;
      }
    }
    __syncthreads();
    if (has_blk) {
      float run[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) run[e] = gcarry[e];
      for (int u = NTB - 1; u >= 0; --u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sGtot[u * DK + cb8 * 8 + e];
          if (u > tb) run[e] += s;
          gcarry[e] += s;
        }
      }
#pragma unroll
      for (int r = 7; r >= 0; --r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ex = __expf(run[e]);
          run[e] += gv[r][e];
          live |= ex != 0.f;
          kv[r][e] *= ex;
        }
      store_blk_rows<E>(sEK + (tb * 8) * LDQ + cb8 * 8, LDQ, kv);
    }
    if (!__syncthreads_or(live)) break;
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w + jj * kWaves;
      if (jb < NJB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const int t = tT * 16 + n16;
          const f32x4 acc = mma_regX<E, NKB>(zero4(), R[jj], sEK + t * LDQ);  // (G^T (e k_t))[j]
          E* dvp = dv + (t0 + t) * Dv + j0 + jb * 16 + 4 * g4;
          store4(dvp, load4(dvp) + acc);
        }
      }
    }
    __syncthreads();
  }
}

template <typename E, int C, int DV, int DKT>
struct CorrectBwdDkLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P;
    const dim3 grid(round_up(n_units, 8) * (a.Dk / DKT));
    hipLaunchKernelGGL((correct_bwd_dk_kernel<E, C, DV, DKT>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};
template <typename E, int C, int DK, int DVT>
struct CorrectBwdDvLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P;
    const dim3 grid(round_up(n_units, 8) * (a.Dv / DVT));
    hipLaunchKernelGGL((correct_bwd_dv_kernel<E, C, DK, DVT>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_correct_bwd_dk(int dtype, int chunk, int dk, int dv) {
  return lookup3<CorrectBwdDkLauncher, Bf16Dv, F32Dv>(dtype, chunk, dv, tile_of(dk));
}
launch_fn lookup_correct_bwd_dv(int dtype, int chunk, int dk, int dv) {
  return lookup3<CorrectBwdDvLauncher, Bf16Dk, F32Dk>(dtype, chunk, dk, tile_of(dv));
}

}  // namespace gla
