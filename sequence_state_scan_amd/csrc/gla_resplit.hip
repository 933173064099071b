// The re-split of flagged units.  The fast local kernels stop a unit at a chunk in which some
// channel decays faster than they can carry, and the exact sub-block kernels redo that unit; they
// are several times slower per token, so one such unit alone would keep its workgroup busy long
// after the rest of the chip has finished.  Instead the flagged units are listed and each is cut
// into X pieces: the state pass gives every piece's end state from a zero start, the scan below
// chains the pieces of each unit (the segment scan of the ZeCO pages, inside one unit), and the
// exact kernels run every piece from its true incoming state (unit_place).
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

namespace {

constexpr int kListThreads = 1024;

// Sum of x over the workgroup; red holds one int per wave.  Every thread gets the sum.
__device__ int block_sum(int x, int* red) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  if (lane_id() == 0) red[wave_id()] = x;
  __syncthreads();
  int s = 0;
  for (int w = 0; w < kListThreads / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

}  // namespace

// One workgroup.  list = {n, X, u_0 .. u_{n-1}}: the first n = min(flagged, R) flagged units in
// unit order, X = the largest power of 2 <= xmax with n X <= R; the listed units' flags are
// cleared (the plain exact pass then skips them and takes only the flagged units beyond R).
__global__ __launch_bounds__(kListThreads) void resplit_list_kernel(int* __restrict__ flags, int* __restrict__ list,
                                                                    int n_units, int R, int xmax) {
  __shared__ int red[kListThreads / 64];
  int c = 0;
  for (int u = threadIdx.x; u < n_units; u += kListThreads) c += flags[u] != 0;
  const int n = min(block_sum(c, red), R);
  int X = xmax;
  while (X > 1 && n * X > R) X >>= 1;
  // rank of each flagged unit: the flagged units before its block of kListThreads, then the
  // flagged lanes before it in its wave, then the flagged lanes of the waves before it
  int base = 0;
  for (int u0 = 0; u0 < n_units && base < n; u0 += kListThreads) {
    const int u = u0 + threadIdx.x;
    const bool f = u < n_units && flags[u] != 0;
    const unsigned long long m = __ballot(f);
    const int lane = lane_id();
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) red[wave_id()] = __popcll(m);
    __syncthreads();
    int waves_before = 0, total = 0;
    for (int w = 0; w < kListThreads / 64; ++w) {
      waves_before += w < wave_id() ? red[w] : 0;
      total += red[w];
    }
    __syncthreads();
    const int rank = base + waves_before + before;
    if (f && rank < n) {
      list[2 + rank] = u;
      flags[u] = 0;
    }
    base += total;
  }
  if (threadIdx.x == 0) {
    list[0] = n;
    list[1] = X;
  }
}

// The segment scan over each listed unit's X pieces, one lane per (unit, state element), in the
// pieces' order (reverse: from the last piece back):
//   carry[first] = hb[u] (zero without hb),  carry[next] = exp(ld[piece]) carry[piece] + state[piece]
// and hout[u] = the value after the unit's last piece.  Nothing to do when X = 1.
__global__ __launch_bounds__(kThreads) void resplit_scan_kernel(const int* __restrict__ list,
                                                                const float* __restrict__ state,
                                                                const float* __restrict__ logdecay,
                                                                const float* __restrict__ hb, float* __restrict__ carry,
                                                                float* __restrict__ hout, int dk, int dv, int reverse) {
  const int n = list[0], X = list[1];
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

hipError_t launch_resplit_list(int* flags, int* list, int n_units, int R, int xmax, hipStream_t stream) {
  hipLaunchKernelGGL(resplit_list_kernel, dim3(1), dim3(kListThreads), 0, stream, flags, list, n_units, R, xmax);
  return hipGetLastError();
}

hipError_t launch_resplit_scan(const int* list, const float* r_state, const float* r_ld, const float* hb,
                               float* r_carry, float* hout, int R, int dk, int dv, int reverse, hipStream_t stream) {
  // at most R / 2 units have pieces to chain (X >= 2); the lanes loop over them, so a small grid
  // will do (and costs little when nothing was flagged)
  const long lanes = (long)(R / 2 > 0 ? R / 2 : 1) * dk * dv;
  const long blocks = (lanes + kThreads - 1) / kThreads;
  const int grid = (int)(blocks < 256 ? blocks : 256);
  hipLaunchKernelGGL(resplit_scan_kernel, dim3(grid), dim3(kThreads), 0, stream, list, r_state, r_ld, hb, r_carry,
                     hout, dk, dv, reverse);
  return hipGetLastError();
}

}  // namespace gla
