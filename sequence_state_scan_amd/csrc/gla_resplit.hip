// The re-split of flagged units.  The fast local kernels stop a unit at a chunk in which some
// channel decays faster than they can carry, and the exact sub-block kernels redo that unit; they
// are several times slower per token, so one such unit alone would keep its workgroup busy long
// after the rest of the chip has finished.  Instead the flagged units are listed and each is cut
// into X pieces: the state pass lists them (resplit_derive) and gives every piece's end state from
// a zero start, the scan below chains the pieces of each unit (the segment scan of the ZeCO pages,
// inside one unit), and the exact kernels run every piece from its true incoming state
// (unit_place).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

// First the listed units' flags are cleared.  Then the segment scan over each listed unit's X
// pieces, one lane per (unit, state element), in the pieces' order (reverse: from the last piece
// back):
//   carry[first] = hb[u] (zero without hb),  carry[next] = exp(ld[piece]) carry[piece] + state[piece]
// and hout[u] = the value after the unit's last piece.  Nothing to scan when X = 1.
__global__ __launch_bounds__(kThreads) void resplit_scan_kernel(const int* __restrict__ list, int* __restrict__ flags,
                                                                const float* __restrict__ state,
                                                                const float* __restrict__ logdecay,
                                                                const float* __restrict__ hb, float* __restrict__ carry,
                                                                float* __restrict__ hout, int dk, int dv, int reverse) {
  const int n = list[0], X = list[1];
  for (int e = blockIdx.x * kThreads + threadIdx.x; e < n; e += gridDim.x * kThreads) flags[list[2 + e]] = 0;
  if (X < 2) return;
  const long st = (long)dk * dv, total = (long)n * st;
  for (long i = (long)blockIdx.x * kThreads + threadIdx.x; i < total; i += (long)gridDim.x * kThreads) {
    const int e = (int)(i / st);
    const long off = i - e * st;
    const int r = (int)(off / dv);
    const long u = list[2 + e];
    float acc = hb ? hb[u * st + off] : 0.f;
    constexpr int NB = 8;  // pieces whose loads are issued before the chain's multiply-adds
    for (int x0 = 0; x0 < X; x0 += NB) {
      float d[NB], y[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const long slot = (long)e * X + (reverse ? X - 1 - (x0 + b) : x0 + b);
        if (x0 + b < X) {
          d[b] = logdecay[slot * dk + r];
          y[b] = state[slot * st + off];
        }
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const long slot = (long)e * X + (reverse ? X - 1 - (x0 + b) : x0 + b);
        if (x0 + b < X) {
          carry[slot * st + off] = acc;
          acc = fmaf(expf(d[b]), acc, y[b]);
        }
      }
    }
    if (hout) hout[u * st + off] = acc;
  }
}

hipError_t launch_resplit_scan(const int* list, int* flags, const float* r_state, const float* r_ld, const float* hb,
                               float* r_carry, float* hout, int R, int dk, int dv, int reverse, hipStream_t stream) {
  // at most R / 2 units have pieces to chain (X >= 2); the lanes loop over them, so a small grid
  // will do (and costs little when nothing was flagged)
  const long lanes = (long)(R / 2 > 0 ? R / 2 : 1) * dk * dv;
  const long blocks = (lanes + kThreads - 1) / kThreads;
  const int grid = (int)(blocks < 256 ? blocks : 256);
  hipLaunchKernelGGL(resplit_scan_kernel, dim3(grid), dim3(kThreads), 0, stream, list, flags, r_state, r_ld, hb,
                     r_carry, hout, dk, dv, reverse);
  return hipGetLastError();
}

}  // namespace gla
