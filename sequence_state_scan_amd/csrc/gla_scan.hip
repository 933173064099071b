// Decay-and-add scan over segments (the All-Scan update of the ZeCO pages, run on one GPU):
//   forward:  carry[0] = h,  carry[p+1] = exp(logdecay[p]) * carry[p] + state[p]
//   reverse:  carry[P-1] = h, carry[p-1] = exp(logdecay[p]) * carry[p] + state[p]
// The state's d_k rows are split into K blocks of d_k/K rows; a row's decay never touches
// another row, so each block is scanned on its own and the result is the same for every K.
// One lane owns one (row, column) element of a block and walks the P segments; consecutive
// lanes own consecutive columns, so every load and store of a wavefront is contiguous.
#include "gla_common.hpp"
#include "gla_kernels.hpp"

namespace gla {

__global__ __launch_bounds__(kThreads) void segment_scan_kernel(
    const float* __restrict__ state, const float* __restrict__ logdecay, const float* __restrict__ hb,
    float* __restrict__ carry, float* __restrict__ hout, int P, int dk, int dv, int K, int reverse,
    int groups_per_block) {
  const int rows = dk / K;
  const long per_blk = (long)rows * dv;
  long b = blockIdx.x;
  const long grp = b % groups_per_block;
  b /= groups_per_block;
  const int kblk = (int)(b % K);
  const long bh = b / K;
  const long e = grp * kThreads + threadIdx.x;
  if (e >= per_blk) return;
  const int r = kblk * rows + (int)(e / dv);
  const int j = (int)(e - (e / dv) * dv);
  const long st = (long)dk * dv;
  const long off = (long)r * dv + j;
  float acc = hb ? hb[bh * st + off] : 0.f;
  if (!reverse) {
    for (int p = 0; p < P; ++p) {
      const long u = bh * P + p;
      carry[u * st + off] = acc;
      acc = fmaf(expf(logdecay[u * dk + r]), acc, state[u * st + off]);
    }
  } else {
    for (int p = P - 1; p >= 0; --p) {
      const long u = bh * P + p;
      carry[u * st + off] = acc;
      acc = fmaf(expf(logdecay[u * dk + r]), acc, state[u * st + off]);
    }
  }
  if (hout) hout[bh * st + off] = acc;
}

hipError_t launch_segment_scan(const float* seg_state, const float* seg_logdecay, const float* h_boundary,
                               float* seg_carry, float* h_out, int BH, int P, int dk, int dv, int K,
                               int reverse, hipStream_t stream) {
  const long per_blk = (long)(dk / K) * dv;
  const int groups = (int)((per_blk + kThreads - 1) / kThreads);
  const dim3 grid((unsigned)((long)BH * K * groups));
  hipLaunchKernelGGL(segment_scan_kernel, grid, dim3(kThreads), 0, stream, seg_state, seg_logdecay,
                     h_boundary, seg_carry, h_out, P, dk, dv, K, reverse, groups);
  return hipGetLastError();
}

}  // namespace gla
