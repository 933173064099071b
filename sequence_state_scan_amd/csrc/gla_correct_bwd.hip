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
//
// SPLIT: a segment is cut into a.S sub-segments of consecutive chunks, one workgroup each.  The
// workgroup of an earlier sub-segment first walks the gate of the chunks after it, from the
// segment's end, with the same prefix sums in the same order as the one-workgroup walk, so its
// running sums, its early stop and so its results are bit for bit those of the whole walk.
// Workgroups are numbered sub-segment first, from the last, so that the last sub-segments of
// every segment, where the correction is live, are dispatched first.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// One workgroup of NW waves per unit.  G is constant over the segment and sits in registers,
// rounded to the element type (the MFMA operand type), in two lane layouts: wave w holds the rows
// c = 16w.. of G (all of d_v) for dk and dg, which contract G over d_v, and the columns of the
// adjacent blocks j = 16 JPW w.. of G (all of d_k) for dv, which contracts it over d_k.  In bf16,
// dk and dv are read and written as merged pairs of 16-column tiles, 16 bytes per lane.  Per live chunk,
// every read of g, k, V and of the outputs to update is issued first; the global state before the
// chunk (for R_n) is read after the chunk is known to be live.
template <typename E, int C, int DK, int DV, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void correct_bwd_kernel(CorrArgs a, int n_units) {
  constexpr int NT = NW * 64;
  constexpr int RI = C / 16, NCG = DK / 4, NI = 16 * NCG;  // strided items of g and k
  constexpr int NVP = C * DV / 8, VPT = ceil_div(NVP, NT);
  constexpr int LDV = lds_ld<E>(DV), LDQ = lds_ld<E>(DK);
  constexpr int NJB = DV / 16, NCB = DK / 16, NTT = C / 16, NKB = DK / 16;
  constexpr int JPW = ceil_div(NJB, NW);
  constexpr bool PAIRS = sizeof(E) == 2;  // dv moves as merged pairs of 16-column tiles
  constexpr bool TPAIRS = PAIRS && NTT % 2 == 0;  // dk moves as merged pairs of 16-token tiles
  static_assert(NI <= NT, "one strided item of g and k per thread");
  static_assert(NCB <= NW, "one 16-row block of G per wave");
  static_assert(JPW == 1 || NJB % NW == 0, "a wave owns JPW column blocks, or none");
  typedef typename Piece4<E>::type piece;

  __shared__ __attribute__((aligned(16))) E sV[C * LDV];   // V [t][j]
  __shared__ __attribute__((aligned(16))) E sEK[C * LDQ];  // exp(r_t) k_t [t][c]

  const int unit = blockIdx.x;
  if (unit >= n_units) return;
  const E* __restrict__ k = static_cast<const E*>(a.k);
  const E* __restrict__ v = static_cast<const E*>(a.v);
  const E* __restrict__ cst = static_cast<const E*>(a.chunk_states);
  const float* __restrict__ g = a.g;
  E* __restrict__ dk = static_cast<E*>(a.dk);
  E* __restrict__ dv = static_cast<E*>(a.dv);
  float* __restrict__ dg = a.dg;
  const int NS = SPLIT ? a.S : 1, nseg = a.BH * a.P;  // sub-segments per segment, segments
  const int sub = SPLIT ? NS - 1 - unit / nseg : 0, seg = SPLIT ? unit - (NS - 1 - sub) * nseg : unit;
  const int L = a.T / a.P;
  const int nchunks = L / C, nsub = nchunks / NS;
  const int bh = seg / a.P, p = seg - bh * a.P;
  const long tok0 = (long)bh * a.T + (long)p * L;
  const long chunk0 = (long)seg * nchunks;
  constexpr long SS = (long)DK * DV;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id(), n16 = l & 15, g4 = l >> 4;
  const bool krole = w < NCB;            // holds rows 16w.. of G
  const bool vrole = w * JPW < NJB;      // holds the columns of G's blocks JPW w..
  // item of a thread: tokens 16r + n16 (r < RI), channels 4cg.. with cg = tid / 16 = 4w + g4: exactly
  // the (t, c) of the lane's dk accumulators below
  const bool has_item = NI == NT || tid < NI;
  const int cg = tid >> 4;

  // G rows: Gr[jb][i] = G[16w + n16][16jb + 4g4 + i];  G columns: Gt[jj][kb][i] = G[16kb + 4g4 + i][16jb + n16]
  // with jb = JPW w + jj
  const float* gp = a.seg_grad + (long)seg * SS;
  piece Gr[NJB], Gt[JPW][NKB];
  int nonzero = 0;
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    const f32x4 x = krole ? load4(gp + (long)(w * 16 + n16) * DV + jb * 16 + 4 * g4) : zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Gr[jb][i] = (E)x[i];
      nonzero |= x[i] != 0.f;
    }
  }
#pragma unroll
  for (int jj = 0; jj < JPW; ++jj) {
    const int jb = w * JPW + jj;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const f32x4 x = vrole ? quad_transpose(load4(gp + (long)(kb * 16 + 4 * g4 + (n16 & 3)) * DV + jb * 16 + (n16 & ~3)))
                            : zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) Gt[jj][kb][i] = (E)x[i];
    }
  }
  if (!__syncthreads_or(nonzero)) return;  // G_p == 0: nothing to add

  float gcarry[4] = {0.f, 0.f, 0.f, 0.f};  // sum of g over the chunks after the current one
  // the gate of the chunks after the sub-segment, from the segment's end, NB chunks' loads in
  // flight at a time
  constexpr int NB = 4;
  const int n_last = (sub + 1) * nsub - 1;  // the sub-segment's last chunk
  if constexpr (SPLIT) {
    for (int n0 = nchunks - 1; n0 > n_last; n0 -= NB) {
      RowsRx4<float, RI> pg[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        if (n0 - i > n_last && has_item) pg[i].load(g + (tok0 + (long)(n0 - i) * C + n16) * DK + cg * 4, 16 * DK);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        if (n0 - i > n_last) {
          float b[RI][4], lam[4];
          chunk_gate_prefix_strided<RI>(pg[i], has_item, b, lam);
          int live = 0;
#pragma unroll
          for (int r = 0; r < RI; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) live |= (has_item ? __expf(gcarry[e] + (lam[e] - b[r][e])) : 0.f) != 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) gcarry[e] += lam[e];
          if (!__syncthreads_or(live)) return;  // the walk stops before the sub-segment
        }
      }
    }
  }
  for (int n = n_last; n >= sub * nsub; --n) {
    const long t0 = tok0 + (long)n * C;
    // ---- every read of the chunk but the state: g, k, V and the outputs to update ----
    RowsRx4<float, RI> pg;
    RowsRx4<E, RI> pk;
    if (has_item) {
      const long off = (t0 + n16) * DK + cg * 4;
      pg.load(g + off, 16 * DK);
      pk.load(k + off, 16 * DK);
    }
    Vec8<E> pv[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pv[i].load(v + (t0 + pc / (DV / 8)) * DV + (pc % (DV / 8)) * 8);
    }
    piece dkprev[NTT];
    f32x4 dgprev[NTT];
    if (krole) {
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) {
        dgprev[tT] = load4(dg + (t0 + tT * 16 + n16) * DK + w * 16 + 4 * g4);
        if constexpr (TPAIRS) {
          // token tiles tT - 1 and tT as one merged pair: lane rows 0 and 2 hold 8 channels of token
          // 16(tT - 1) + n16, rows 1 and 3 those of token 16 tT + n16
          if (tT & 1)
            unmerge_pair(*reinterpret_cast<const bf16x8*>(dk + (t0 + 16 * (tT - 1 + (g4 & 1)) + n16) * DK + w * 16 +
                                                          8 * (g4 >> 1)),
                         dkprev[tT - 1], dkprev[tT]);
        } else {
          dkprev[tT] = load_piece(dk + (t0 + tT * 16 + n16) * DK + w * 16 + 4 * g4);
        }
      }
    }
    piece dvprev[JPW][NTT];
    if (vrole) {
#pragma unroll
      for (int sT = 0; sT < NTT; ++sT) {
        if constexpr (PAIRS && JPW == 2) {
          unmerge_pair(*reinterpret_cast<const bf16x8*>(dv + (t0 + sT * 16 + n16) * DV + w * 32 + pair_col(g4)),
                       dvprev[0][sT], dvprev[1][sT]);
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj)
            dvprev[jj][sT] = load_piece(dv + (t0 + sT * 16 + n16) * DV + (w * JPW + jj) * 16 + 4 * g4);
        }
      }
    }
    // ---- exp(r_t), r_t = sum of g over the tokens after t up to the segment's end; exp(r) k -> LDS ----
    float er[RI][4], lam[4];
    int live = 0;
    {
      float b[RI][4];
      chunk_gate_prefix_strided<RI>(pg, has_item, b, lam);
#pragma unroll
      for (int r = 0; r < RI; ++r) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          er[r][e] = has_item ? __expf(gcarry[e] + (lam[e] - b[r][e])) : 0.f;
          live |= er[r][e] != 0.f;
          x[e] = pk.at(r, e) * er[r][e];
        }
        if (has_item) store4(sEK + (16 * r + n16) * LDQ + cg * 4, x);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int pc = tid + NT * i;
      if (NVP % NT == 0 || pc < NVP) pv[i].store(sV + (pc / (DV / 8)) * LDV + (pc % (DV / 8)) * 8);
    }
    if (!__syncthreads_or(live)) break;
    // ---- dk and dg (rows 16w.. of G) ----
    if (krole) {
      // R_n = rowsum(S_{n-1} * G) for c = 16w + n16
      const long roff = (long)(w * 16 + n16) * DV + 4 * g4;
      float part = 0.f;
      if (n > 0) {
        const E* st = cst + (chunk0 + n - 1) * SS;
        if constexpr (NJB % 2 == 0) {
#pragma unroll
          for (int m = 0; m < NJB / 2; ++m) {
            piece s0, s1;
            load_state_pair<E, NJB>(st, w, m, state_lane_row(n16, g4), s0, s1);
            part += piece_dot(s0, Gr[2 * m]) + piece_dot(s1, Gr[2 * m + 1]);
          }
        } else {
#pragma unroll
          for (int jb = 0; jb < NJB; ++jb)
            part += piece_dot(load_state_piece<E, NJB>(st, w, jb, state_lane_row(n16, g4)), Gr[jb]);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const f32x4 x = load4(a.seg_in + (long)seg * SS + roff + jb * 16);
          piece sp;
#pragma unroll
          for (int i = 0; i < 4; ++i) sp[i] = (E)x[i];
          part += piece_dot(sp, Gr[jb]);
        }
      }
      part = sum_over_g4(part);
      // dk[t][c] += exp(r_t) (G v_t)[c];  dg[t][c] += E_n R_n + sum_{s < t in the chunk} k_s dk'_s
      f32x4 before;  // E_n R_n plus the sums of the earlier row blocks, c = 16w + 4g4 + i
      f32x4 dkn[2];  // the new dk of the current pair of token tiles
#pragma unroll
      for (int i = 0; i < 4; ++i)
        before[i] = __expf(gcarry[i] + lam[i]) * __shfl(part, (l & ~15) | (4 * g4 + i));
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) {
        const int t = tT * 16 + n16;
        f32x4 acc = mma_regX_e<E, NJB>(zero4(), Gr, sV + t * LDV);  // (G v_t)[c]
        f32x4 ddk, kd, d;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ddk[i] = acc[i] * er[tT][i];
          kd[i] = pk.at(tT, i) * ddk[i];
          const float incl = seg_scan_incl<16>(kd[i]);
          d[i] = dgprev[tT][i] + before[i] + (incl - kd[i]);
          before[i] += seg_last<16>(incl);
        }
        const long go = (t0 + t) * DK + w * 16 + 4 * g4;
        store4(dg + go, d);
        if constexpr (TPAIRS) {
          dkn[tT & 1] = widen(dkprev[tT]) + ddk;
          if (tT & 1)
            *reinterpret_cast<bf16x8*>(dk + (t0 + 16 * (tT - 1 + (g4 & 1)) + n16) * DK + w * 16 + 8 * (g4 >> 1)) =
                merge_pair(to_bf16x4(dkn[0]), to_bf16x4(dkn[1]));
        } else {
          store4(dk + go, widen(dkprev[tT]) + ddk);
        }
      }
    }
    // ---- dv (columns of G) ----
    if (vrole) {
#pragma unroll
      for (int sT = 0; sT < NTT; ++sT) {
        // dv^T[j][s] += sum_c G^T[j][c] (exp(r_s) k_s)[c]
        f32x4 acc[JPW];
#pragma unroll
        for (int jj = 0; jj < JPW; ++jj)
          acc[jj] = mma_regX_e<E, NKB>(widen(dvprev[jj][sT]), Gt[jj], sEK + (sT * 16 + n16) * LDQ);
        if constexpr (PAIRS && JPW == 2) {
          *reinterpret_cast<bf16x8*>(dv + (t0 + sT * 16 + n16) * DV + w * 32 + pair_col(g4)) =
              merge_pair(to_bf16x4(acc[0]), to_bf16x4(acc[1]));
        } else {
#pragma unroll
          for (int jj = 0; jj < JPW; ++jj) store4(dv + (t0 + sT * 16 + n16) * DV + (w * JPW + jj) * 16 + 4 * g4, acc[jj]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) gcarry[e] += lam[e];
    __syncthreads();
  }
}

template <typename E, int C, int DK, int DV>
struct CorrectBwdLauncher {
  static hipError_t run(const void* pa, hipStream_t s) {
    const CorrArgs& a = *static_cast<const CorrArgs*>(pa);
    const int n_units = a.BH * a.P * a.S;
    if (a.S > 1)
      hipLaunchKernelGGL((correct_bwd_kernel<E, C, DK, DV, 8, true>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    else
      hipLaunchKernelGGL((correct_bwd_kernel<E, C, DK, DV, 8, false>), dim3(n_units), dim3(8 * 64), 0, s, a, n_units);
    return hipGetLastError();
  }
};

launch_fn lookup_correct_bwd(int dtype, int chunk, int dk, int dv) {
  return lookup_cdd<CorrectBwdLauncher, Bf16CorrChunks>(dtype, chunk, dk, dv);
}

}  // namespace gla
