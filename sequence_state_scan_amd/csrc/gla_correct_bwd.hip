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
// registers (wave w owns the 16-row blocks cb = w, w+4, ...) and feeds the MFMA A operand.  Every
// global read of a chunk is issued before its writes (one memory round trip per chunk).
template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void correct_bwd_dk_kernel(CorrArgs a, int n_units) {
  constexpr int DKT = DK < 64 ? DK : 64, NT = DK / DKT;
  constexpr int NTG = C / 4, NCG = DKT / 8, NI = NTG * NCG;
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, kThreads);
  constexpr int LDV = DV + kPad, LDL = DKT + 4;
  constexpr int NJB = DV / 16, NCB = DKT / 16, NTT = C / 16;
  constexpr int CPW = ceil_div(NCB, kWaves);
  static_assert(NI <= kThreads, "one 4x8 item per thread");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sV[C * LDV];      // V [t][j]
  __shared__ __attribute__((aligned(16))) float sE[C * LDL];  // exp(r_t) [t][c]
  __shared__ __attribute__((aligned(16))) float sKD[C * LDL]; // k * delta-dk [t][c]
  __shared__ float sR[DKT];                                   // R_n

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
  constexpr long SS = (long)DK * DV;
  const int c0 = tile * DKT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  // item of g and dg: tokens 4tg..4tg+3, slice channels 8cg..8cg+7
  const bool has_item = tid < NI;
  const int tg = tid % NTG, cg = tid / NTG;

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

  float gcarry[8];  // sum of g over the chunks after the current one, up to the segment's end
#pragma unroll
  for (int e = 0; e < 8; ++e) gcarry[e] = 0.f;
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    // every read of this chunk before its writes: g, V, dk, k and the global state before the
    // chunk here, dg once the chunk is known to be live
    Rows4x8<float> pg, pdg;
    if (has_item) pg.load(g + (t0 + tg * 4) * DK + c0 + cg * 8, DK);
    Vec8<E> pv[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + kThreads * i;
      if (NVP % kThreads == 0 || pc < NVP) pv[i].load(v + (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
    piece dkprev[CPW][NTT], kk[CPW][NTT], Sp[CPW][NJB];
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * kWaves;
      if (cb < NCB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const long go = (t0 + tT * 16 + n16) * DK + c0 + cb * 16 + 4 * g4;
          dkprev[cc][tT] = load_piece(dk + go);
          kk[cc][tT] = load_piece(k + go);
        }
        const long roff = (long)(c0 + cb * 16 + n16) * DV + 4 * g4;
        if (n > 0) {
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
    }
    // exp(r_t), r_t = sum of g over the tokens after t up to the segment's end
    float lam[8];
    int live = 0;
    {
      float b[4][8];
      chunk_gate_prefix<NTG>(pg, has_item, b, lam);
      if (has_item) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[e] = __expf(gcarry[e] + (lam[e] - b[r][e]));
            live |= x[e] != 0.f;
          }
          store8(sE + (tg * 4 + r) * LDL + cg * 8, x);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + kThreads * i;
      if (NVP % kThreads == 0 || pc < NVP) pv[i].store(sV + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
    }
    if (!__syncthreads_or(live)) break;
    if (has_item) pdg.load(dg + (t0 + tg * 4) * DK + c0 + cg * 8, DK);
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int cb = w + cc * kWaves;
      if (cb < NCB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const int t = tT * 16 + n16;
          f32x4 acc = mma_regX<E, NJB>(zero4(), R[cc], sV + t * LDV);  // (G v_t)[c]
          acc *= load4(sE + t * LDL + cb * 16 + 4 * g4);
          store4(dk + (t0 + t) * DK + c0 + cb * 16 + 4 * g4, widen(dkprev[cc][tT]) + acc);
          store4(sKD + t * LDL + cb * 16 + 4 * g4, widen(kk[cc][tT]) * acc);
        }
        float part = 0.f;  // R_n = rowsum(S_{n-1} * G)
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) part += piece_dot(Sp[cc][jb], R[cc][jb]);
        part = sum_over_g4(part);
        if (g4 == 0) sR[cb * 16 + n16] = part;
      }
    }
    __syncthreads();
    // dg[t] += E_n R_n + sum_{s < t in the chunk} k_s delta-dk_s, E_n = exp(sum of g from the
    // chunk's first token to the segment's end)
    {
      float xs[4][8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (has_item) load8(sKD + (tg * 4 + r) * LDL + cg * 8, xs[r]);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[r][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = xs[r][e];
          xs[r][e] = run;
          run += x;
        }
        const float excl = seg_prev<NTG>(seg_scan_incl<NTG>(run));
        const float base = has_item ? __expf(gcarry[e] + lam[e]) * sR[cg * 8 + e] + excl : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[r][e] += base;
      }
      if (has_item)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float outv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) outv[e] = pdg.at(r, e) + xs[r][e];
          store8(dg + (t0 + tg * 4 + r) * DK + c0 + cg * 8, outv);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) gcarry[e] += lam[e];
    __syncthreads();
  }
}

// dv: one workgroup per (unit, DVT-wide slice of d_v).  G^T[j][:] for the slice in registers.
template <typename E, int C, int DK, int DV>
__global__ __launch_bounds__(kThreads) void correct_bwd_dv_kernel(CorrArgs a, int n_units) {
  constexpr int DVT = DV < 64 ? DV : 64, NT = DV / DVT;
  constexpr int NTG = C / 4, NCG = DK / 8, NI = NTG * NCG;
  constexpr int LDQ = DK + kPad;
  constexpr int NJB = DVT / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, kWaves);
  static_assert(NI <= kThreads, "one 4x8 item per thread");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sEK[2][C * LDQ];  // exp(r_t) k_t [t][c], by chunk parity

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
  const bool has_item = tid < NI;
  const int tg = tid % NTG, cg = tid / NTG;

  // G^T slice: R[jj][kb][i] = G[16kb + 4g4 + i][j0 + 16jb + n16]
  const float* gp = a.seg_grad + (long)unit * DK * DV;
  f32x4 R[JPW][NKB];
  int nonzero = 0;
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int jb = w + jj * kWaves;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const f32x4 x = jb < NJB ? load4(gp + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + j0 + jb * 16 + (n16 & ~3))
                               : zero4();
      R[jj][kb] = quad_transpose(x);
#pragma unroll
      for (int i = 0; i < 4; ++i) nonzero |= x[i] != 0.f;
    }
  }
  if (!__syncthreads_or(nonzero)) return;

  float gcarry[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gcarry[e] = 0.f;
  const int nchunks = L / C;
  for (int n = nchunks - 1; n >= 0; --n) {
    const long t0 = tok0 + (long)n * C;
    const int par = n & 1;
    Rows4x8<float> pg;
    Rows4x8<E> pk;
    if (has_item) {
      pg.load(g + (t0 + tg * 4) * DK + cg * 8, DK);
      pk.load(k + (t0 + tg * 4) * DK + cg * 8, DK);
    }
    piece dvprev[JPW][NTT];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w + jj * kWaves;
      if (jb < NJB)
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT)
          dvprev[jj][tT] = load_piece(dv + (t0 + tT * 16 + n16) * DV + j0 + jb * 16 + 4 * g4);
    }
    int live = 0;
    {
      float b[4][8], lam[8];
      chunk_gate_prefix<NTG>(pg, has_item, b, lam);
      if (has_item) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float ex = __expf(gcarry[e] + (lam[e] - b[r][e]));
            live |= ex != 0.f;
            x[e] = pk.at(r, e) * ex;
          }
          store8(&sEK[par][(tg * 4 + r) * LDQ + cg * 8], x);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) gcarry[e] += lam[e];
    }
    if (!__syncthreads_or(live)) break;
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w + jj * kWaves;
      if (jb < NJB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          const int t = tT * 16 + n16;
          const f32x4 acc = mma_regX<E, NKB>(widen(dvprev[jj][tT]), R[jj], &sEK[par][t * LDQ]);  // + G^T (e k_t)
          store4(dv + (t0 + t) * DV + j0 + jb * 16 + 4 * g4, acc);
        }
      }
    }
  }
}

template <typename E, int C, int DK, int DV>
struct CorrectBwdDkLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P;
    constexpr int NT = DK / (DK < 64 ? DK : 64);
    const dim3 grid(round_up(n_units, 8) * NT);
    hipLaunchKernelGGL((correct_bwd_dk_kernel<E, C, DK, DV>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};
template <typename E, int C, int DK, int DV>
struct CorrectBwdDvLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P;
    constexpr int NT = DV / (DV < 64 ? DV : 64);
    const dim3 grid(round_up(n_units, 8) * NT);
    hipLaunchKernelGGL((correct_bwd_dv_kernel<E, C, DK, DV>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_correct_bwd_dk(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<CorrectBwdDkLauncher>(dtype, chunk, dk, dv);
}
launch_fn lookup_correct_bwd_dv(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<CorrectBwdDvLauncher>(dtype, chunk, dk, dv);
}

}  // namespace gla
