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
  // NB segments at a time: their loads are independent of the chain, so all of them are issued
  // before the dependent multiply-adds (the chain's arithmetic and order are unchanged)
  constexpr int NB = 8;
  for (int p0 = 0; p0 < P; p0 += NB) {
    float d[NB], x[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int p = reverse ? P - 1 - (p0 + i) : p0 + i;
      if (p0 + i < P) {
        const long u = bh * P + p;
        d[i] = logdecay[u * dk + r];
        x[i] = state[u * st + off];
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int p = reverse ? P - 1 - (p0 + i) : p0 + i;
      if (p0 + i < P) {
        const long u = bh * P + p;
        carry[u * st + off] = acc;
        acc = fmaf(expf(d[i]), acc, x[i]);
      }
    }
  }
  if (hout) hout[bh * st + off] = acc;
}

// The all-gather ordering of the same scan (the LASP2 pattern the ZeCO key-facts page compares
// against, rendered on one GPU): every output combines the local states it depends on directly,
// with no chain between outputs,
//   forward: carry[p] = sum_{q<p} exp(sum_{q<r<p} ld[r]) state[q] + exp(sum_{r<p} ld[r]) h,
//            h_out = the same with p = P
//   reverse: carry[p] = sum_{q>p} exp(sum_{p<r<q} ld[r]) state[q] + exp(sum_{r>p} ld[r]) h,
//            h_out = the same with p = -1
// O(P^2) state reads instead of O(P), every output independent.  One lane per (output, element);
// the decay exponent is accumulated in the log domain along the walk.
__global__ __launch_bounds__(kThreads) void segment_scan_allgather_kernel(
    const float* __restrict__ state, const float* __restrict__ logdecay, const float* __restrict__ hb,
    float* __restrict__ carry, float* __restrict__ hout, int P, int dk, int dv, int reverse, int groups_per_out) {
  const long st = (long)dk * dv;
  long b = blockIdx.x;
  const long grp = b % groups_per_out;
  b /= groups_per_out;
  const int oi = (int)(b % (P + 1));  // output index: 0..P-1 carries, P h_out
  const long bh = b / (P + 1);
  const long e = grp * kThreads + threadIdx.x;
  if (e >= st) return;
  if (oi == P && !hout) return;
  const int r = (int)(e / dv);
  float acc = 0.f, s = 0.f;
  if (!reverse) {
    const int p = oi;  // combines segments p-1, p-2, .., 0, then h
    for (int q = p - 1; q >= 0; --q) {
      const long u = bh * P + q;
      acc = fmaf(expf(s), state[u * st + e], acc);
      s += logdecay[u * dk + r];
    }
  } else {
    const int p = oi == P ? -1 : oi;  // combines segments p+1, .., P-1, then h
    for (int q = p + 1; q < P; ++q) {
      const long u = bh * P + q;
      acc = fmaf(expf(s), state[u * st + e], acc);
      s += logdecay[u * dk + r];
    }
  }
  if (hb) acc = fmaf(expf(s), hb[bh * st + e], acc);
  if (oi == P) hout[bh * st + e] = acc;
  else carry[(bh * P + oi) * st + e] = acc;
}

hipError_t launch_segment_scan_allgather(const float* seg_state, const float* seg_logdecay, const float* h_boundary,
                                         float* seg_carry, float* h_out, int BH, int P, int dk, int dv, int reverse,
                                         hipStream_t stream) {
  const long st = (long)dk * dv;
  const int groups = (int)((st + kThreads - 1) / kThreads);
  const dim3 grid((unsigned)((long)BH * (P + 1) * groups));
  hipLaunchKernelGGL(segment_scan_allgather_kernel, grid, dim3(kThreads), 0, stream, seg_state, seg_logdecay,
                     h_boundary, seg_carry, h_out, P, dk, dv, reverse, groups);
  return hipGetLastError();
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

// A segment's summed log-gates from its S sub-segments' (in sub-segment order, as the local
// kernels sum them): one lane per (segment, channel).
__global__ __launch_bounds__(kThreads) void sum_logdecay_kernel(const float* __restrict__ sub_ld,
                                                                float* __restrict__ seg_ld, long n, int S, int dk) {
  const long i = (long)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const long u = i / dk, c = i - u * dk;
  float sum = 0.f;
  for (int s = 0; s < S; ++s) sum += sub_ld[(u * S + s) * dk + c];
  seg_ld[i] = sum;
}

hipError_t launch_sum_logdecay(const float* sub_ld, float* seg_ld, int n_units, int S, int dk, hipStream_t stream) {
  const long n = (long)n_units * dk;
  hipLaunchKernelGGL(sum_logdecay_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, stream,
                     sub_ld, seg_ld, n, S, dk);
  return hipGetLastError();
}

}  // namespace gla
