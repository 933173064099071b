// Host-visible declarations shared by the HIP translation units of libgla.so: argument blocks,
// the launcher table and the list of shapes kernels are built for.
#pragma once
#include <hip/hip_runtime_api.h>

#include "gla.h"

#include <type_traits>
#include <utility>

namespace gla {

struct FwdArgs {  // gla_chunk_fwd
  const void *q, *k, *v;
  const float* g;
  void* o;
  void* chunk_states;  // [B][H][T/C][dk][dv], element type = dtype
  float *seg_state, *seg_logdecay;
  int* flags;  // [BH * P * S] per-unit flags in the workspace: 1 = recompute with the exact kernel
  int BH, T, Dk, Dv, P, chunk;
  // Each segment is cut into S sub-segments of T/(P S) tokens, one workgroup each (S = 1: none).
  // init: [BH * P * S][Dk][Dv] state entering each sub-segment, counted from its segment's start
  // (read for sub-segments s > 0); sub_state / sub_ld: the state pass's outputs, the state at the
  // end of each sub-segment from a zero start and the sub-segment's summed log-gates.
  int S;
  const float* init;
  float *sub_state, *sub_ld;
  // Re-split of the units the fast kernel flagged (list non-null; see unit_place): R slots, one
  // workgroup each, over the listed units' pieces (at most xmax per unit).  r_init: [R][Dk][Dv]
  // state entering each piece, counted from its segment's start; r_state / r_ld: the state pass's
  // outputs per piece.  The state pass over the pieces writes the list (resplit_derive).
  int* list;
  int R, xmax;
  const float* r_init;
  float *r_state, *r_ld;
  // from_in = 1: the segments' incoming states are known (the ordering that runs the state pass
  // and the scan before the local pass).  init is then the GLOBAL state entering every unit, its
  // segment's first sub-segment included, so outputs and chunk states come out global, and the
  // segment-level outputs (seg_state, seg_logdecay) are neither needed nor written.
  int from_in;
  // reach = 1 (the state pass only, not with list): walk each sub-segment from its last chunk,
  // weighting token t by exp(summed log-gates after t), and stop once every channel's summed
  // log-gates are below kReachCut; sub_ld then holds the sum over the chunks walked.
  int reach;
};

struct BwdArgs {  // gla_chunk_bwd
  const void *q, *k, *v;
  const float* g;
  const void* dO;
  const void* chunk_states;  // global states after every chunk
  const float* seg_in;
  void *dq, *dk, *dv;
  float *dg, *seg_dstate;
  int* flags;  // as in FwdArgs
  int BH, T, Dk, Dv, P, chunk;
  // Sub-segments as in FwdArgs.  init: [BH * P * S][Dk][Dv] gradient w.r.t. the state leaving each
  // sub-segment from the later sub-segments of its segment (read for s < S - 1); sub_state, sub_ld:
  // the state-gradient pass's outputs, each sub-segment's gradient w.r.t. its incoming state from
  // its own outputs, and its summed log-gates.
  int S;
  const float* init;
  float *sub_state, *sub_ld;
  // Re-split of flagged units as in FwdArgs; r_init: gradient w.r.t. the state leaving each piece
  // from the rest of its segment.
  int* list;
  int R, xmax;
  const float* r_init;
  float *r_state, *r_ld;
  // from_in = 1: init is the GLOBAL gradient w.r.t. the state leaving every unit, its segment's
  // last sub-segment included (the later segments' share), so dk, dv and dg come out global;
  // seg_dstate is neither needed nor written.
  int from_in;
  // reach = 1 (the state-gradient pass only, not with list): walk each sub-segment from its first
  // chunk, weighting token t by exp(summed log-gates from the sub-segment's start through t), and
  // stop once every channel's sum is below kReachCut; sub_ld then holds the sum over the chunks
  // walked.
  int reach;
};

// gla_chunk_fwd with the sub-segment split capped at max_split (0: no cap), the workspace already
// checked to hold workspace_size bytes for that cap.  With seg_in non-null it is
// gla_chunk_fwd_from: every segment starts from seg_in[p] (seg_state, seg_logdecay unused).
gla_status chunk_fwd_capped(const void* q, const void* k, const void* v, const float* g, const float* seg_in, void* o,
                            void* chunk_states, float* seg_state, float* seg_logdecay, int B, int H, int T, int dk,
                            int dv, int chunk, int P, int dtype, void* workspace, size_t workspace_size,
                            int max_split, void* stream);

struct CorrArgs {  // gla_segment_correct
  const void *q, *k, *v;
  const float *g, *seg_in, *seg_grad;
  void *o, *chunk_states, *dk, *dv;
  float* dg;
  int BH, T, Dk, Dv, P;
  int S;  // sub-segments per segment, one workgroup each (a power of 2 dividing the chunks)
};

typedef hipError_t (*launch_fn)(const void* args, hipStream_t stream);

// Units (b, h, segment) the static scratch of gla_chunk_fwd_noalloc holds flags for (256 KiB).
constexpr int kStaticUnits = 65536;

// The calling thread's last-error record of the C ABI (gla_last_error): set it, and read its status.
gla_status set_error(gla_status s, const char* fmt, ...);
gla_status last_status();

// Compile-time shape lists.  bf16: the MFMA K step is 32, so every contracted length
// (chunk, d_k, d_v) is a multiple of 32.  f32 kernels exist for small heads only.
template <int... Vs> struct IntList {};
using Bf16Chunks = IntList<32, 64>;          // fast local kernels (the MFMA K step is 32 tokens)
using Bf16CorrChunks = IntList<16, 32, 64>;  // corrections (their products contract over d_k, d_v)
using Bf16Dk = IntList<32, 64, 128>;
using Bf16Dv = IntList<32, 64, 128, 256>;
using F32Chunks = IntList<16, 32, 64>;
using F32Dk = IntList<16, 32>;
using F32Dv = IntList<16, 32>;

template <typename F, int... Vs>
inline bool dispatch_int(int v, IntList<Vs...>, F&& f) {
  return ((v == Vs ? (f(std::integral_constant<int, Vs>{}), true) : false) || ...);
}

// Per translation unit lookups; nullptr when no kernel exists for the shape.
// dtype: 0 = f32, 1 = bf16.
launch_fn lookup_fwd_local(int dtype, int chunk, int dk, int dv);
launch_fn lookup_correct_fwd(int dtype, int chunk, int dk, int dv);
launch_fn lookup_bwd(int dtype, int chunk, int dk, int dv);
launch_fn lookup_correct_bwd(int dtype, int chunk, int dk, int dv);
// The exact sub-block kernels (any chunk in {16, 32, 64}; chunk is an argument).  With flags
// non-null only the units whose flag is 1 are processed, else every unit.
launch_fn lookup_fwd_exact(int dtype, int dk, int dv);
launch_fn lookup_bwd_exact(int dtype, int dk, int dv);
// The state passes over sub-segments (forward: sub_state, sub_ld; backward: sub_state).
launch_fn lookup_fwd_state(int dtype, int chunk, int dk, int dv);
launch_fn lookup_bwd_state(int dtype, int chunk, int dk, int dv);

hipError_t launch_segment_scan(const float* seg_state, const float* seg_logdecay, const float* h_boundary,
                               float* seg_carry, float* h_out, int BH, int P, int dk, int dv, int K,
                               int reverse, hipStream_t stream);
// The scan of the re-split (list = {n, X, u_0 .. u_{n-1}}, written by the state pass over the
// pieces): clears the listed units' flags, so that the plain exact pass skips them and takes only
// the flagged units beyond R; then, when X > 1, the segment scan over each listed unit's X pieces,
// starting from hb[u] (null: zero) and writing the end value to hout[u] (null: not written).
hipError_t launch_resplit_scan(const int* list, int* flags, const float* r_state, const float* r_ld, const float* hb,
                               float* r_carry, float* hout, int R, int dk, int dv, int reverse, hipStream_t stream);

// seg_ld[u][c] = sum over s < S of sub_ld[u][s][c]: a segment's summed log-gates from its
// sub-segments', for n_units segments of dk channels.
hipError_t launch_sum_logdecay(const float* sub_ld, float* seg_ld, int n_units, int S, int dk, hipStream_t stream);

hipError_t launch_segment_scan_allgather(const float* seg_state, const float* seg_logdecay, const float* h_boundary,
                                         float* seg_carry, float* h_out, int BH, int P, int dk, int dv, int reverse,
                                         hipStream_t stream);

// Generic lookup over (dtype, dk, dv): Launcher<E, DK, DV>::run.
template <template <typename, int, int> class Launcher>
inline launch_fn lookup_dd(int dtype, int dk, int dv) {
  launch_fn r = nullptr;
  if (dtype == 1) {
    dispatch_int(dk, Bf16Dk{}, [&](auto a) {
      dispatch_int(dv, Bf16Dv{}, [&](auto b) { r = &Launcher<__bf16, a.value, b.value>::run; });
    });
  } else if (dtype == 0) {
    dispatch_int(dk, F32Dk{}, [&](auto a) {
      dispatch_int(dv, F32Dv{}, [&](auto b) { r = &Launcher<float, a.value, b.value>::run; });
    });
  }
  return r;
}

// Generic lookup over (dtype, chunk, dk, dv): Launcher<E, C, DK, DV>::run.
template <template <typename, int, int, int> class Launcher, class Bf16C = Bf16Chunks>
inline launch_fn lookup_cdd(int dtype, int chunk, int dk, int dv) {
  launch_fn r = nullptr;
  if (dtype == 1) {
    dispatch_int(chunk, Bf16C{}, [&](auto c) {
      dispatch_int(dk, Bf16Dk{}, [&](auto a) {
        dispatch_int(dv, Bf16Dv{}, [&](auto b) { r = &Launcher<__bf16, c.value, a.value, b.value>::run; });
      });
    });
  } else if (dtype == 0) {
    dispatch_int(chunk, F32Chunks{}, [&](auto c) {
      dispatch_int(dk, F32Dk{}, [&](auto a) {
        dispatch_int(dv, F32Dv{}, [&](auto b) { r = &Launcher<float, c.value, a.value, b.value>::run; });
      });
    });
  }
  return r;
}

}  // namespace gla
