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
// dk x dv) lives in accumulator registers for the whole segment: wave w owns the 16-column
// blocks jb = w, w+NW, ...  After every chunk the state is also written out (chunk_states,
// element type E): the local chunk states the correction turns into global ones and the
// backward reads.
//
// Per chunk: (1) the gate's running sum is taken with a shuffle scan across the lanes that hold
// one 8-channel column (4 tokens per lane), q/k are scaled and every tile is staged in LDS, and
// the next chunk's q, k, g, v are requested into registers; (2) the intra-chunk scores;
// (3) outputs and the state update on MFMA.  The requests of (1) are in flight during (2)-(3).
template <typename E, int C, int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void fwd_local_kernel(FwdArgs a, int n_units) {
  constexpr int NT = NW * 64;
  constexpr int NTG = C / 4, NCG = DK / 8, NI = NTG * NCG, RT = NT / 2;
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDQ = DK + kPad, LDV = DV + kPad, LDT = C + kPad;
  constexpr int NJB = DV / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, NW);
  constexpr int KS = Mma<E>::KSTEP;
  static_assert(NI <= RT, "one 4x8 item of q (and one of k) per loader thread");

  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];   // Qbar [t][c]
  __shared__ __attribute__((aligned(16))) E sK[C * LDQ];   // Kbar [s][c]
  __shared__ __attribute__((aligned(16))) E sKt[C * LDQ];  // Ktil [s][c]
  __shared__ __attribute__((aligned(16))) E sV[C * LDV];   // V    [s][j]
  __shared__ __attribute__((aligned(16))) E sA[C * LDT];   // A    [t][s], masked
  __shared__ float sLamE[DK];                              // exp(lam) per channel

  const int unit = blockIdx.x;
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const float* __restrict__ g = a.g;
  E* __restrict__ o = static_cast<E*>(a.o);
  E* __restrict__ cst = static_cast<E*>(a.chunk_states);
  const int L = a.T / a.P;
  const int nchunks = L / C;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const long chunk0 = (long)unit * nchunks;

  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool krole = tid >= RT;
  const int rt = krole ? tid - RT : tid;
  const bool has_item = rt < NI;
  const int tg = rt % NTG, cg = rt / NTG;
  const E* __restrict__ xsrc = krole ? k : q;

  Rows4x8<float> pg;
  Rows4x8<E> px;
  Vec8<E> pv[VPT];
  auto prefetch = [&](int n) {
    const long t0 = tok0 + (long)n * C;
    if (has_item) {
      pg.load(g + (t0 + tg * 4) * DK + cg * 8, DK);
      px.load(xsrc + (t0 + tg * 4) * DK + cg * 8, DK);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pv[i].load(v + (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
  };

  f32x4 S[JPW][NKB];
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) S[jj][kb] = zero4();
  float ldsum[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ldsum[e] = 0.f;

  prefetch(0);
  for (int n = 0; n < nchunks; ++n) {
    const long t0 = tok0 + (long)n * C;
    // ---- (1) gate prefix sums, scaled q / k, V -> LDS; request the next chunk ----
    {
      float b[4][8], lam[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          run += has_item ? pg.at(r, e) : 0.f;
          b[r][e] = run;
        }
        const float incl = seg_scan_incl<NTG>(run);
        const float excl = seg_prev<NTG>(incl);
        lam[e] = seg_last<NTG>(incl);
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r][e] += excl;
      }
      if (has_item) {
        if (!krole) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = px.at(r, e) * __expf(b[r][e]);
            store8(sQ + (tg * 4 + r) * LDQ + cg * 8, x);
          }
          if (tg == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              sLamE[cg * 8 + e] = __expf(lam[e]);
              ldsum[e] += lam[e];
            }
          }
        } else {
          float el[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) el[e] = __expf(lam[e]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float xb[8], xt[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              xb[e] = px.at(r, e) * __expf(-b[r][e]);
              xt[e] = xb[e] * el[e];
            }
            store8(sK + (tg * 4 + r) * LDQ + cg * 8, xb);
            store8(sKt + (tg * 4 + r) * LDQ + cg * 8, xt);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int pc = tid + NT * i;
        if (NVP % NT == 0 || pc < NVP) pv[i].store(sV + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the next chunk's loads after this chunk's staging
    if (n + 1 < nchunks) prefetch(n + 1);
    __syncthreads();
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
    E* cs = cst + (chunk0 + n) * (long)DK * DV;
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w + jj * NW;
      if (jb < NJB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          f32x4 acc = zero4();
          const int ke = round_up((tT + 1) * 16, KS) < C ? round_up((tT + 1) * 16, KS) : C;
          acc = mma<E, true, false>(acc, sV + jb * 16, LDV, sA + tT * 16 * LDT, LDT, 0, ke);
          acc = mma_regX<E, NKB>(acc, S[jj], sQ + (tT * 16 + n16) * LDQ);
          store4(o + (t0 + tT * 16 + n16) * DV + jb * 16 + 4 * g4, acc);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) S[jj][kb][i] *= sLamE[kb * 16 + 4 * g4 + i];
          S[jj][kb] = mma<E, true, true>(S[jj][kb], sKt + kb * 16, LDQ, sV + jb * 16, LDV, 0, C);
          // lane (n16 = 4m + r) stores row 16kb + 4g4 + r, columns 16jb + 4m .. +3
          store4(cs + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + jb * 16 + (n16 & ~3), quad_transpose(S[jj][kb]));
        }
      }
    }
    __syncthreads();
  }

  // ---- segment results: local end state (float32) and log cumulative decay ----
  float* st = a.seg_state + (long)unit * DK * DV;
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int jb = w + jj * NW;
    if (jb < NJB)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        store4(st + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + jb * 16 + (n16 & ~3), quad_transpose(S[jj][kb]));
  }
  if (!krole && has_item && tg == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a.seg_logdecay[(long)unit * DK + cg * 8 + e] = ldsum[e];
  }
}

// Correction of segment p's local results with its incoming global state S_in[p]:
//   o_t              += (q_t * a_t) . S_in[p],   a_t = exp(sum of g from the segment start to t)
//   chunk_states[n]  += diag(a at the end of chunk n) S_in[p]
// One workgroup per (unit, d_v slice); S_in's slice sits in registers in the accumulator layout
// and feeds the MFMA A operand directly.  With g <= 0, a_t only decreases: once every a_t of a
// chunk is exactly 0.0f, so are all later ones (and the chunk-end decays), and the loop stops.
template <typename E, int C, int DK, int DVT>
__global__ __launch_bounds__(kThreads) void correct_fwd_kernel(CorrArgs a, int n_units) {
  constexpr int NTB = C / 8, NCB8 = DK / 8, NQB = NTB * NCB8;
  constexpr int LDQ = DK + kPad;
  constexpr int NJB = DVT / 16, NKB = DK / 16, NTT = C / 16;
  constexpr int JPW = ceil_div(NJB, kWaves);
  static_assert(NQB <= kThreads, "one 8x8 block of q per loader thread");

  __shared__ __attribute__((aligned(16))) E sQ[C * LDQ];  // q * a   [t][c]
  __shared__ float sGtot[NTB * DK];
  __shared__ float sAend[DK];                              // a at the chunk's last token

  const int NT = a.Dv / DVT;
  int unit, tile;
  xcd_map(blockIdx.x, NT, unit, tile);
  if (unit >= n_units) return;
  const E* __restrict__ q = static_cast<const E*>(a.q);
  const float* __restrict__ g = a.g;
  E* __restrict__ o = static_cast<E*>(a.o);
  E* __restrict__ cst = static_cast<E*>(a.chunk_states);
  const int Dv = a.Dv;
  const int L = a.T / a.P;
  const int nchunks = L / C;
  const int bh = unit / a.P, p = unit - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const long chunk0 = (long)unit * nchunks;
  const int j0 = tile * DVT;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool has_blk = tid < NQB;
  const int tb = tid / NCB8, cb = tid - (tid / NCB8) * NCB8;

  // incoming state slice, accumulator layout: R[jj][kb][i] = S_in[16kb + 4g4 + i][j0 + 16jb + n16]
  f32x4 R[JPW][NKB];
  const float* sin = a.seg_in + (long)unit * DK * Dv;
  int nonzero = 0;
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int jb = w + jj * kWaves;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        R[jj][kb][i] = jb < NJB ? sin[(long)(kb * 16 + 4 * g4 + i) * Dv + j0 + jb * 16 + n16] : 0.f;
        nonzero |= R[jj][kb][i] != 0.f;
      }
  }
  if (!__syncthreads_or(nonzero)) return;  // zero incoming state: nothing to add

  float carry[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) carry[e] = 0.f;
  for (int n = 0; n < nchunks; ++n) {
    const long t0 = tok0 + (long)n * C;
    float gv[8][8], xv[8][8];
    int live = 0;
    if (has_blk) {
      load_blk<float>(gv, g + (t0 + tb * 8) * DK + cb * 8, DK);
      load_blk<E>(xv, q + (t0 + tb * 8) * DK + cb * 8, DK);
#pragma unroll
      for (int r = 1; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[r][e] += gv[r - 1][e];
#pragma unroll
      for (int e = 0; e < 8; ++e) sGtot[tb * DK + cb * 8 + e] = gv[7][e];
    }
    __syncthreads();
    if (has_blk) {
      float pre[8], tot[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { pre[e] = carry[e]; tot[e] = 0.f; }
      for (int u = 0; u < NTB; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float s = sGtot[u * DK + cb * 8 + e];
          if (u < tb) pre[e] += s;
          tot[e] += s;
        }
      }
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float av = __expf(gv[r][e] + pre[e]);
          live |= av != 0.f;
          xv[r][e] *= av;
        }
      store_blk_rows<E>(sQ + (tb * 8) * LDQ + cb * 8, LDQ, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) carry[e] += tot[e];
      if (tb == 0)
#pragma unroll
        for (int e = 0; e < 8; ++e) sAend[cb * 8 + e] = __expf(carry[e]);
    }
    if (!__syncthreads_or(live)) break;  // every a_t of this chunk (and all later ones) is 0
    E* cs = cst + (chunk0 + n) * (long)DK * Dv;
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int jb = w + jj * kWaves;
      if (jb < NJB) {
#pragma unroll
        for (int tT = 0; tT < NTT; ++tT) {
          f32x4 acc = mma_regX<E, NKB>(zero4(), R[jj], sQ + (tT * 16 + n16) * LDQ);
          E* op = o + (t0 + tT * 16 + n16) * Dv + j0 + jb * 16 + 4 * g4;
          const f32x4 prev = load4(op);
          store4(op, prev + acc);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = kb * 16 + 4 * g4 + i;
            E* sp = cs + (long)c * Dv + j0 + jb * 16 + n16;
            *sp = (E)((float)*sp + sAend[c] * R[jj][kb][i]);
          }
      }
    }
    __syncthreads();
  }
}

template <typename E, int C, int DK, int DV>
struct FwdLocalLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const FwdArgs& a = *static_cast<const FwdArgs*>(pa);
    const int n_units = a.BH * a.P;
    hipLaunchKernelGGL((fwd_local_kernel<E, C, DK, DV, 8>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};

template <typename E, int C, int DK, int DVT>
struct CorrectFwdLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P;
    const dim3 grid(round_up(n_units, 8) * (a.Dv / DVT));
    hipLaunchKernelGGL((correct_fwd_kernel<E, C, DK, DVT>), grid, dim3(kThreads), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_fwd_local(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<FwdLocalLauncher>(dtype, chunk, dk, dv);
}
launch_fn lookup_correct_fwd(int dtype, int chunk, int dk, int dv) {
  return lookup3<CorrectFwdLauncher, Bf16Dk, F32Dk>(dtype, chunk, dk, tile_of(dv));
}

}  // namespace gla
