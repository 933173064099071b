// C ABI of libgla.so (declared in include/gla.h): host-side argument checks, then kernel
// launches on the caller's stream.  Every check runs before the first HIP call, so a rejected
// call enqueues nothing and touches no device.
#include "gla.h"

#include <cstdarg>
#include <cstdio>
#include <string>

#include "gla_kernels.hpp"

namespace {

thread_local std::string g_last_error;
thread_local gla_status g_last_status = GLA_OK;

gla_status vfail(gla_status s, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_last_error = buf;
  g_last_status = s;
  return s;
}

gla_status fail(gla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(s, fmt, ap);
  va_end(ap);
  return s;
}

gla_status ok() {
  g_last_error.clear();
  g_last_status = GLA_OK;
  return GLA_OK;
}

bool in_list(int v, std::initializer_list<int> l) {
  for (int x : l)
    if (x == v) return true;
  return false;
}

bool shape_listed(int dtype, int dk, int dv, int chunk) {
  if (dtype == GLA_BF16)
    return in_list(chunk, {16, 32, 64}) && in_list(dk, {32, 64, 128}) && in_list(dv, {32, 64, 128, 256});
  if (dtype == GLA_F32)
    return in_list(chunk, {16, 32, 64}) && in_list(dk, {16, 32}) && in_list(dv, {16, 32});
  return false;
}

struct Kernels {
  gla::launch_fn fwd, corr_fwd, bwd, corr_bwd;  // fwd and bwd: the fast local kernels (null for bf16 chunk 16)
  gla::launch_fn fwd_exact, bwd_exact;          // the exact sub-block kernels
  gla::launch_fn fwd_state, bwd_state;          // the state passes over sub-segments (with the fast kernels)
};

bool find_kernels(int dtype, int dk, int dv, int chunk, Kernels* k) {
  if (!shape_listed(dtype, dk, dv, chunk)) return false;
  k->fwd = gla::lookup_fwd_local(dtype, chunk, dk, dv);
  k->corr_fwd = gla::lookup_correct_fwd(dtype, chunk, dk, dv);
  k->bwd = gla::lookup_bwd(dtype, chunk, dk, dv);
  k->corr_bwd = gla::lookup_correct_bwd(dtype, chunk, dk, dv);
  k->fwd_exact = gla::lookup_fwd_exact(dtype, dk, dv);
  k->bwd_exact = gla::lookup_bwd_exact(dtype, dk, dv);
  k->fwd_state = gla::lookup_fwd_state(dtype, chunk, dk, dv);
  k->bwd_state = gla::lookup_bwd_state(dtype, chunk, dk, dv);
  return (k->fwd != nullptr) == (k->bwd != nullptr) && (k->fwd != nullptr) == (k->fwd_state != nullptr) &&
         (k->fwd != nullptr) == (k->bwd_state != nullptr) && k->corr_fwd && k->corr_bwd && k->fwd_exact &&
         k->bwd_exact;
}

// Sub-segments per segment.  One workgroup runs a (b, h, segment) unit, and at most one fits on a
// CU, so with fewer than 256 units most of the chip would idle: each segment is then cut into S
// sub-segments (a power of two, each of at least 2 chunks) until B*H*P*S reaches 256.  A state
// pass gives every sub-segment's end state (backward: its state gradient), the segment scan
// combines them inside each segment, and the local pass starts every sub-segment from its true
// incoming state (gradient), so its outputs are the ones the unsplit segment would give.  Only
// the fast kernels split (bf16 chunk 16 runs unsplit).
constexpr long long kFillUnits = 256;
int split_factor(int B, int H, int T, int P, int chunk, const Kernels& k) {
  if (!k.fwd) return 1;
  const long long units = (long long)B * H * P;
  const int nch = T / P / chunk;
  int S = 1;
  while (units * S < kFillUnits && nch % (2 * S) == 0 && nch / (2 * S) >= 2) S *= 2;
  return S;
}

// Sub-segments of the corrections, where the segments alone leave CUs idle: as many as fill the
// chip, one chunk each at least.  (Cutting finer was slower: a sub-segment's gate walk over the
// chunks before it grows with the number of cuts.)
int correct_split(int B, int H, int T, int P, int chunk) {
  const long long units = (long long)B * H * P;
  const int nch = T / P / chunk;
  int S = 1;
  while (units * S < kFillUnits && nch % (2 * S) == 0) S *= 2;
  return S;
}

// The re-split of flagged units.  A unit the fast kernel flags is redone by the exact sub-block
// kernels, several times slower per token: alone it would keep one workgroup busy long after the
// rest of the chip is done.  So the flagged units are listed on the device and each is cut into X
// pieces of at least 2 chunks, with X chosen there from how many were flagged, so that the pieces
// fill R slots (workgroups): a state pass over the pieces, the scan over each unit's pieces, then
// the exact kernels run every piece from its true incoming state.  Flagged units beyond R run
// whole, as before.  xmax: the most pieces a unit of S-split segments allows.
int resplit_xmax(int T, int P, int S, int chunk) {
  const int nch = T / P / S / chunk;
  int X = 1;
  while (nch % (2 * X) == 0 && nch / (2 * X) >= 2) X *= 2;
  return X;
}
int resplit_slots(int B, int H, int T, int P, int S, int chunk, const Kernels& k) {
  if (!k.fwd) return 0;  // every unit runs the exact kernels, split as the units are
  const int x = resplit_xmax(T, P, S, chunk);
  if (x < 2) return 0;
  const long long slots = (long long)B * H * P * S * x;
  return (int)(slots < kFillUnits ? slots : kFillUnits);
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of gla_chunk_fwd / gla_chunk_bwd, in this order: one int flag per unit (b, h, segment,
// sub-segment); with S > 1 the sub-segments' states from the state pass, their summed log-gates,
// and the scan's incoming states (forward) or gradients (backward), all float32; with R > 0 the
// re-split's list (2 + R ints) and per slot the same three float32 arrays.
struct Workspace {
  size_t flags, sub_state, sub_ld, carry, list, r_state, r_ld, r_carry, total;
};
Workspace workspace_layout(int B, int H, int P, int dk, int dv, int S, int R) {
  const size_t u = (size_t)B * H * P * S, ss = (size_t)dk * dv * sizeof(float);
  Workspace w{};
  w.flags = 0;
  size_t off = align256(u * sizeof(int));
  if (S > 1) {
    w.sub_state = off;
    off += align256(u * ss);
    w.sub_ld = off;
    off += align256(u * dk * sizeof(float));
    w.carry = off;
    off += align256(u * ss);
  }
  if (R > 0) {
    w.list = off;
    off += align256((size_t)(2 + R) * sizeof(int));
    w.r_state = off;
    off += align256((size_t)R * ss);
    w.r_ld = off;
    off += align256((size_t)R * dk * sizeof(float));
    w.r_carry = off;
    off += align256((size_t)R * ss);
  }
  w.total = off;
  return w;
}

// The schedule a workspace allows: S sub-segments per segment and R re-split slots.
struct Schedule {
  int S, R;
};
Schedule fastest_schedule(int B, int H, int T, int chunk, int P, const Kernels& k, int max_split) {
  int S = split_factor(B, H, T, P, chunk, k);
  if (max_split > 0 && S > max_split) S = max_split;
  return {S, resplit_slots(B, H, T, P, S, chunk, k)};
}
size_t workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int P, const Kernels& k) {
  const Schedule f = fastest_schedule(B, H, T, chunk, P, k, 0);
  return workspace_layout(B, H, P, dk, dv, f.S, f.R).total;
}

// The fastest schedule a workspace of `bytes` allows: a smaller workspace first gives up the
// re-split, then halves S and tries the re-split again, down to S = 1 with no re-split (one flag
// per unit); S = 0 if not even that fits.
Schedule fitting_schedule(int B, int H, int T, int dk, int dv, int chunk, int P, const Kernels& k, int max_split,
                          size_t bytes) {
  for (int S = fastest_schedule(B, H, T, chunk, P, k, max_split).S; S >= 1; S /= 2) {
    const int R = resplit_slots(B, H, T, P, S, chunk, k);
    if (workspace_layout(B, H, P, dk, dv, S, R).total <= bytes) return {S, R};
    if (workspace_layout(B, H, P, dk, dv, S, 0).total <= bytes) return {S, 0};
  }
  return {0, 0};
}

// Shape checks shared by the chunked entry points.
gla_status check_shape(const char* fn, int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                       Kernels* kern) {
  if (B < 1 || H < 1 || T < 1 || P < 1 || dk < 1 || dv < 1 || chunk < 1)
    return fail(GLA_ERR_INVALID_ARG, "%s: B, H, T, dk, dv, chunk and P must be >= 1", fn);
  if (dtype != GLA_F32 && dtype != GLA_BF16) return fail(GLA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  if (T % P != 0) return fail(GLA_ERR_INVALID_ARG, "%s: T=%d is not a multiple of P=%d", fn, T, P);
  if ((T / P) % chunk != 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: segment length %d is not a multiple of chunk=%d", fn, T / P, chunk);
  const long long units = (long long)B * H * P;
  if (units * 4 > (1LL << 30)) return fail(GLA_ERR_INVALID_ARG, "%s: B*H*P=%lld is too large", fn, units);
  if (!find_kernels(dtype, dk, dv, chunk, kern))
    return fail(GLA_ERR_UNSUPPORTED, "%s: no kernel for dtype=%s dk=%d dv=%d chunk=%d", fn,
                dtype == GLA_BF16 ? "bf16" : "f32", dk, dv, chunk);
  return GLA_OK;
}

gla_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(GLA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// The state passes of gla_chunk_state / gla_chunk_dstate: the kernels of `chunk`, or where there
// are none (bf16 chunk 16 runs only the exact kernels) those of the longest chunk that divides the
// segments (the state does not depend on the chunk length beyond rounding).  Returns the chunk
// length used, 0 if none will do.
int state_pass_chunk(int dtype, int dk, int dv, int chunk, int seg_len, gla::launch_fn* fwd_state,
                     gla::launch_fn* bwd_state) {
  for (int c : {chunk, 64, 32}) {
    if (seg_len % c != 0) continue;
    *fwd_state = gla::lookup_fwd_state(dtype, c, dk, dv);
    *bwd_state = gla::lookup_bwd_state(dtype, c, dk, dv);
    if (*fwd_state && *bwd_state) return c;
  }
  return 0;
}

// Sub-segments of a state pass: as many as the workspace holds, up to the count that fills the chip.
int state_pass_split(int B, int H, int T, int dk, int dv, int chunk, int P, size_t bytes) {
  const long long units = (long long)B * H * P;
  const int nch = T / P / chunk;
  int S = 1;
  while (units * S < kFillUnits && nch % (2 * S) == 0 && nch / (2 * S) >= 2 &&
         workspace_layout(B, H, P, dk, dv, 2 * S, 0).total <= bytes)
    S *= 2;
  return S;
}

// gla_chunk_state (which == GLA_FWD: seg_state, seg_logdecay from k, v, g) and gla_chunk_dstate
// (GLA_BWD: seg_dstate from q, g, do).
gla_status state_pass_run(int which, const void* q, const void* k, const void* v, const float* g, const void* do_,
                          float* out_state, float* out_ld, int B, int H, int T, int dk, int dv, int chunk, int P,
                          int dtype, void* workspace, size_t workspace_size, void* stream) {
  const char* fn = which == GLA_FWD ? "gla_chunk_state" : "gla_chunk_dstate";
  Kernels kern;
  gla_status st = check_shape(fn, B, H, T, dk, dv, chunk, P, dtype, &kern);
  if (st != GLA_OK) return st;
  if (which == GLA_FWD ? (!k || !v || !g || !out_state || !out_ld) : (!q || !g || !do_ || !out_state))
    return fail(GLA_ERR_INVALID_ARG, which == GLA_FWD ? "%s: k, v, g, seg_state and seg_logdecay must be non-null"
                                                      : "%s: q, g, do and seg_dstate must be non-null", fn);
  const void* ins[] = {q, k, v, g, do_};
  for (const void* p : ins)
    if (p && (p == out_state || p == out_ld || p == workspace))
      return fail(GLA_ERR_INVALID_ARG, "%s: outputs and the workspace must not alias inputs", fn);
  gla::launch_fn fwd_state = nullptr, bwd_state = nullptr;
  const int cs = state_pass_chunk(dtype, dk, dv, chunk, T / P, &fwd_state, &bwd_state);
  if (!cs)
    return fail(GLA_ERR_UNSUPPORTED, "%s: no state-pass kernel for dtype=%s dk=%d dv=%d and segments of %d tokens",
                fn, dtype == GLA_BF16 ? "bf16" : "f32", dk, dv, T / P);
  const int S = state_pass_split(B, H, T, dk, dv, cs, P, workspace ? workspace_size : 0);
  const Workspace lay = workspace_layout(B, H, P, dk, dv, S, 0);
  char* ws = static_cast<char*>(workspace);
  float* sub_state = S > 1 ? reinterpret_cast<float*>(ws + lay.sub_state) : out_state;
  float* sub_ld = S > 1 ? reinterpret_cast<float*>(ws + lay.sub_ld) : out_ld;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int units = B * H * P;
  if (which == GLA_FWD) {
    gla::FwdArgs a{};
    a.k = k;
    a.v = v;
    a.g = g;
    a.BH = B * H;
    a.T = T;
    a.Dk = dk;
    a.Dv = dv;
    a.P = P;
    a.chunk = cs;
    a.S = S;
    a.sub_state = sub_state;
    a.sub_ld = sub_ld;
    a.reach = 1;  // from each sub-segment's end, as far as its decay reaches
    st = launched(fn, fwd_state(&a, s));
  } else {
    gla::BwdArgs a{};
    a.q = q;
    a.g = g;
    a.dO = do_;
    a.BH = B * H;
    a.T = T;
    a.Dk = dk;
    a.Dv = dv;
    a.P = P;
    a.chunk = cs;
    a.S = S;
    a.sub_state = sub_state;
    a.sub_ld = S > 1 ? sub_ld : nullptr;  // the segments' log decays come from gla_chunk_state
    a.reach = 1;                          // from each sub-segment's start, as far as its decay reaches
    st = launched(fn, bwd_state(&a, s));
  }
  if (st != GLA_OK || S == 1) return st;
  // the scan over each segment's sub-segments, from zero at its start (end): its end value is the
  // segment's state (gradient)
  float* carry = reinterpret_cast<float*>(ws + lay.carry);
  st = launched(fn, gla::launch_segment_scan(sub_state, sub_ld, nullptr, carry, out_state, units, S, dk, dv, 1,
                                             which == GLA_FWD ? 0 : 1, s));
  if (st != GLA_OK || which != GLA_FWD) return st;
  return launched(fn, gla::launch_sum_logdecay(sub_ld, out_ld, units, S, dk, s));
}

}  // namespace

namespace gla {
gla_status set_error(gla_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(s, fmt, ap);
  va_end(ap);
  return s;
}
gla_status last_status() { return g_last_status; }
}  // namespace gla

extern "C" {

int gla_supported(int dtype, int dk, int dv, int chunk) {
  Kernels k;
  return find_kernels(dtype, dk, dv, chunk, &k) ? 1 : 0;
}

const char* gla_status_string(gla_status s) {
  switch (s) {
    case GLA_OK: return "GLA_OK";
    case GLA_ERR_INVALID_ARG: return "GLA_ERR_INVALID_ARG";
    case GLA_ERR_UNSUPPORTED: return "GLA_ERR_UNSUPPORTED";
    case GLA_ERR_HIP: return "GLA_ERR_HIP";
  }
  return "unknown gla_status";
}

const char* gla_last_error(void) { return g_last_error.c_str(); }

size_t gla_workspace_size(int which, int B, int H, int T, int dk, int dv, int chunk, int P, int dtype) {
  if (which != GLA_FWD && which != GLA_BWD) {
    fail(GLA_ERR_INVALID_ARG, "gla_workspace_size: unknown call %d", which);
    return 0;
  }
  Kernels kern;
  if (check_shape("gla_workspace_size", B, H, T, dk, dv, chunk, P, dtype, &kern) != GLA_OK) return 0;
  ok();
  return workspace_bytes(B, H, T, dk, dv, chunk, P, kern);
}

gla_status gla_chunk_fwd(const void* q, const void* k, const void* v, const float* g, void* o,
                         void* chunk_states, float* seg_state, float* seg_logdecay, int B, int H, int T,
                         int dk, int dv, int chunk, int P, int dtype, void* workspace, size_t workspace_size,
                         void* stream) {
  return gla::chunk_fwd_capped(q, k, v, g, nullptr, o, chunk_states, seg_state, seg_logdecay, B, H, T, dk, dv, chunk,
                               P, dtype, workspace, workspace_size, 0, stream);
}

gla_status gla_chunk_fwd_from(const void* q, const void* k, const void* v, const float* g, const float* seg_in,
                              void* o, void* chunk_states, int B, int H, int T, int dk, int dv, int chunk, int P,
                              int dtype, void* workspace, size_t workspace_size, void* stream) {
  if (!seg_in) return fail(GLA_ERR_INVALID_ARG, "gla_chunk_fwd_from: seg_in must be non-null");
  return gla::chunk_fwd_capped(q, k, v, g, seg_in, o, chunk_states, nullptr, nullptr, B, H, T, dk, dv, chunk, P,
                               dtype, workspace, workspace_size, 0, stream);
}

}  // extern "C"

gla_status gla::chunk_fwd_capped(const void* q, const void* k, const void* v, const float* g, const float* seg_in,
                                 void* o, void* chunk_states, float* seg_state, float* seg_logdecay, int B, int H,
                                 int T, int dk, int dv, int chunk, int P, int dtype, void* workspace,
                                 size_t workspace_size, int max_split, void* stream) {
  const bool from = seg_in != nullptr;
  const char* fn = from ? "gla_chunk_fwd_from" : "gla_chunk_fwd";
  Kernels kern;
  gla_status st = check_shape(fn, B, H, T, dk, dv, chunk, P, dtype, &kern);
  if (st != GLA_OK) return st;
  if (from) {
    if (!q || !k || !v || !g || !o)  // chunk_states may be NULL (forward only)
      return fail(GLA_ERR_INVALID_ARG, "%s: q, k, v, g, seg_in and o must be non-null", fn);
  } else if (!q || !k || !v || !g || !o || !seg_state || !seg_logdecay) {  // chunk_states may be NULL
    return fail(GLA_ERR_INVALID_ARG, "%s: q, k, v, g, o, seg_state and seg_logdecay must be non-null", fn);
  }
  const void* ins[] = {q, k, v, g, seg_in};
  for (const void* p : ins)
    if (p && (p == o || p == chunk_states || p == workspace))
      return fail(GLA_ERR_INVALID_ARG, "%s: outputs and the workspace must not alias inputs", fn);
  const Schedule sch = workspace ? fitting_schedule(B, H, T, dk, dv, chunk, P, kern, max_split, workspace_size)
                                 : Schedule{0, 0};
  const int S = sch.S;
  if (S == 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: the workspace needs at least %zu bytes (one int per unit; "
                "gla_workspace_size gives the size for the fastest schedule), got %zu", fn,
                workspace_layout(B, H, P, dk, dv, 1, 0).total, workspace ? workspace_size : (size_t)0);
  const Workspace lay = workspace_layout(B, H, P, dk, dv, S, sch.R);
  char* ws = static_cast<char*>(workspace);
  gla::FwdArgs a{q, k, v, g, o, chunk_states, seg_state, seg_logdecay, reinterpret_cast<int*>(ws + lay.flags),
                 B * H, T, dk, dv, P, chunk, S, from ? seg_in : nullptr, nullptr, nullptr};
  a.from_in = from ? 1 : 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (S > 1) {
    // state pass over the sub-segments, then the scan over them inside each segment: the state
    // entering each sub-segment (from zero at the segment's start, or from seg_in[p]) and, as its
    // end value, the segment's local end state
    a.sub_state = reinterpret_cast<float*>(ws + lay.sub_state);
    a.sub_ld = reinterpret_cast<float*>(ws + lay.sub_ld);
    float* carry = reinterpret_cast<float*>(ws + lay.carry);
    a.init = nullptr;
    st = launched(fn, kern.fwd_state(&a, s));
    if (st != GLA_OK) return st;
    st = launched(fn, gla::launch_segment_scan(a.sub_state, a.sub_ld, seg_in, carry, seg_state, B * H * P, S, dk,
                                               dv, 1, 0, s));
    if (st != GLA_OK) return st;
    a.init = carry;
  }
  if (kern.fwd) {  // the fast kernel, then the exact one for the units it flagged
    st = launched(fn, kern.fwd(&a, s));
    if (st != GLA_OK) return st;
    if (sch.R > 0) {
      // the state pass over the flagged units' pieces (it lists them) and the scan over each
      // unit's pieces (from the unit's incoming state; with S = 1 its end value is the segment's)
      int* list = reinterpret_cast<int*>(ws + lay.list);
      float* r_carry = reinterpret_cast<float*>(ws + lay.r_carry);
      a.list = list;
      a.R = sch.R;
      a.xmax = resplit_xmax(T, P, S, chunk);
      a.r_init = r_carry;
      a.r_state = reinterpret_cast<float*>(ws + lay.r_state);
      a.r_ld = reinterpret_cast<float*>(ws + lay.r_ld);
      st = launched(fn, kern.fwd_state(&a, s));
      if (st != GLA_OK) return st;
      st = launched(fn, gla::launch_resplit_scan(list, a.flags, a.r_state, a.r_ld, a.init, r_carry,
                                                 S > 1 || from ? nullptr : seg_state, sch.R, dk, dv, 0, s));
      if (st != GLA_OK) return st;
    }
  } else {
    a.flags = nullptr;  // every unit
  }
  return launched(fn, kern.fwd_exact(&a, s));
}

extern "C" {

gla_status gla_segment_scan(const float* seg_state, const float* seg_logdecay, const float* h_boundary,
                            float* seg_carry, float* h_out, int B, int H, int P, int dk, int dv, int K,
                            int reverse, void* stream) {
  const char* fn = "gla_segment_scan";
  if (B < 1 || H < 1 || P < 1 || dk < 1 || dv < 1)
    return fail(GLA_ERR_INVALID_ARG, "%s: B, H, P, dk and dv must be >= 1", fn);
  if (K < 1 || K > dk || dk % K != 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: K=%d must divide dk=%d", fn, K, dk);
  if (reverse != 0 && reverse != 1) return fail(GLA_ERR_INVALID_ARG, "%s: reverse must be 0 or 1", fn);
  if (!seg_state || !seg_logdecay || !seg_carry)
    return fail(GLA_ERR_INVALID_ARG, "%s: seg_state, seg_logdecay and seg_carry must be non-null", fn);
  if (seg_carry == seg_state) return fail(GLA_ERR_INVALID_ARG, "%s: seg_carry must not alias seg_state", fn);
  const long long blocks = (long long)B * H * K * (((long long)(dk / K) * dv + 255) / 256);
  if (blocks > 0x7fffffffLL) return fail(GLA_ERR_INVALID_ARG, "%s: problem too large", fn);
  return launched(fn, gla::launch_segment_scan(seg_state, seg_logdecay, h_boundary, seg_carry, h_out, B * H, P,
                                               dk, dv, K, reverse, static_cast<hipStream_t>(stream)));
}

gla_status gla_segment_scan_allgather(const float* seg_state, const float* seg_logdecay, const float* h_boundary,
                                      float* seg_carry, float* h_out, int B, int H, int P, int dk, int dv, int reverse,
                                      void* stream) {
  const char* fn = "gla_segment_scan_allgather";
  if (B < 1 || H < 1 || P < 1 || dk < 1 || dv < 1)
    return fail(GLA_ERR_INVALID_ARG, "%s: B, H, P, dk and dv must be >= 1", fn);
  if (reverse != 0 && reverse != 1) return fail(GLA_ERR_INVALID_ARG, "%s: reverse must be 0 or 1", fn);
  if (!seg_state || !seg_logdecay || !seg_carry)
    return fail(GLA_ERR_INVALID_ARG, "%s: seg_state, seg_logdecay and seg_carry must be non-null", fn);
  if (seg_carry == seg_state) return fail(GLA_ERR_INVALID_ARG, "%s: seg_carry must not alias seg_state", fn);
  const long long blocks = (long long)B * H * (P + 1) * (((long long)dk * dv + 255) / 256);
  if (blocks > 0x7fffffffLL) return fail(GLA_ERR_INVALID_ARG, "%s: problem too large", fn);
  return launched(fn, gla::launch_segment_scan_allgather(seg_state, seg_logdecay, h_boundary, seg_carry, h_out,
                                                         B * H, P, dk, dv, reverse, static_cast<hipStream_t>(stream)));
}

gla_status gla_segment_correct(int mode, const void* q, const void* k, const void* v, const float* g,
                               const float* seg_in, const float* seg_grad, void* o, void* chunk_states, void* dk_,
                               void* dv_, float* dg, int B, int H, int T, int dk, int dv, int chunk, int P,
                               int dtype, void* stream) {
  const char* fn = "gla_segment_correct";
  if (mode != GLA_FWD && mode != GLA_BWD) return fail(GLA_ERR_INVALID_ARG, "%s: unknown mode %d", fn, mode);
  Kernels kern;
  gla_status st = check_shape(fn, B, H, T, dk, dv, chunk, P, dtype, &kern);
  if (st != GLA_OK) return st;
  gla::CorrArgs a{q, k, v, g, seg_in, seg_grad, o, chunk_states, dk_, dv_, dg, B * H, T, dk, dv, P,
                  correct_split(B, H, T, P, chunk)};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == GLA_FWD) {
    if (!q || !g || !seg_in || !o)  // chunk_states may be NULL (forward only)
      return fail(GLA_ERR_INVALID_ARG, "%s(GLA_FWD): q, g, seg_in and o must be non-null", fn);
    return launched(fn, kern.corr_fwd(&a, s));
  }
  if (!k || !v || !g || !seg_in || !seg_grad || !chunk_states || !dk_ || !dv_ || !dg)
    return fail(GLA_ERR_INVALID_ARG,
                "%s(GLA_BWD): k, v, g, seg_in, seg_grad, chunk_states, dk, dv and dg must be non-null", fn);
  return launched(fn, kern.corr_bwd(&a, s));
}

}  // extern "C"

namespace {

// gla_chunk_bwd, or with seg_grad non-null gla_chunk_bwd_from: every segment's backward starts from
// seg_grad[p] at its end (seg_dstate unused).
gla_status chunk_bwd_run(const void* q, const void* k, const void* v, const float* g, const void* do_,
                         const void* chunk_states, const float* seg_in, const float* seg_grad, void* dq, void* dk_,
                         void* dv_, float* dg, float* seg_dstate, int B, int H, int T, int dk, int dv, int chunk,
                         int P, int dtype, void* workspace, size_t workspace_size, void* stream) {
  const bool from = seg_grad != nullptr;
  const char* fn = from ? "gla_chunk_bwd_from" : "gla_chunk_bwd";
  Kernels kern;
  gla_status st = check_shape(fn, B, H, T, dk, dv, chunk, P, dtype, &kern);
  if (st != GLA_OK) return st;
  if (!q || !k || !v || !g || !do_ || !chunk_states || !seg_in || !dq || !dk_ || !dv_ || !dg || (!from && !seg_dstate))
    return fail(GLA_ERR_INVALID_ARG, "%s: every pointer argument must be non-null", fn);
  const void* ins[] = {q, k, v, g, do_, chunk_states, seg_in, seg_grad};
  for (const void* p : ins)
    if (p && (p == dq || p == dk_ || p == dv_ || p == dg || p == seg_dstate || p == workspace))
      return fail(GLA_ERR_INVALID_ARG, "%s: outputs and the workspace must not alias inputs", fn);
  const Schedule sch = workspace ? fitting_schedule(B, H, T, dk, dv, chunk, P, kern, 0, workspace_size)
                                 : Schedule{0, 0};
  const int S = sch.S;
  if (S == 0)
    return fail(GLA_ERR_INVALID_ARG, "%s: the workspace needs at least %zu bytes (one int per unit; "
                "gla_workspace_size gives the size for the fastest schedule), got %zu", fn,
                workspace_layout(B, H, P, dk, dv, 1, 0).total, workspace ? workspace_size : (size_t)0);
  const Workspace lay = workspace_layout(B, H, P, dk, dv, S, sch.R);
  char* ws = static_cast<char*>(workspace);
  gla::BwdArgs a{q, k, v, g, do_, chunk_states, seg_in, dq, dk_, dv_, dg, from ? nullptr : seg_dstate,
                 reinterpret_cast<int*>(ws + lay.flags), B * H, T, dk, dv, P, chunk, S, from ? seg_grad : nullptr,
                 nullptr, nullptr};
  a.from_in = from ? 1 : 0;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (S > 1) {
    // state-gradient pass over the sub-segments, then the reverse scan over them inside each
    // segment: the gradient w.r.t. the state leaving each sub-segment from the rest of its segment
    // (and from the later segments, seg_grad[p], with from) and, as its end value, the segment's
    // gradient w.r.t. its incoming state
    a.sub_state = reinterpret_cast<float*>(ws + lay.sub_state);
    a.sub_ld = reinterpret_cast<float*>(ws + lay.sub_ld);
    float* carry = reinterpret_cast<float*>(ws + lay.carry);
    a.init = nullptr;
    st = launched(fn, kern.bwd_state(&a, s));
    if (st != GLA_OK) return st;
    st = launched(fn, gla::launch_segment_scan(a.sub_state, a.sub_ld, seg_grad, carry, from ? nullptr : seg_dstate,
                                               B * H * P, S, dk, dv, 1, 1, s));
    if (st != GLA_OK) return st;
    a.init = carry;
  }
  if (kern.bwd) {  // the fast kernel, then the exact one for the units it flagged
    st = launched(fn, kern.bwd(&a, s));
    if (st != GLA_OK) return st;
    if (sch.R > 0) {
      // the state-gradient pass over the flagged units' pieces (it lists them) and the reverse
      // scan over each unit's pieces (with S = 1 its end value is the segment's)
      int* list = reinterpret_cast<int*>(ws + lay.list);
      float* r_carry = reinterpret_cast<float*>(ws + lay.r_carry);
      a.list = list;
      a.R = sch.R;
      a.xmax = resplit_xmax(T, P, S, chunk);
      a.r_init = r_carry;
      a.r_state = reinterpret_cast<float*>(ws + lay.r_state);
      a.r_ld = reinterpret_cast<float*>(ws + lay.r_ld);
      st = launched(fn, kern.bwd_state(&a, s));
      if (st != GLA_OK) return st;
      st = launched(fn, gla::launch_resplit_scan(list, a.flags, a.r_state, a.r_ld, a.init, r_carry,
                                                 S > 1 || from ? nullptr : seg_dstate, sch.R, dk, dv, 1, s));
      if (st != GLA_OK) return st;
    }
  } else {
    a.flags = nullptr;  // every unit
  }
  return launched(fn, kern.bwd_exact(&a, s));
}

}  // namespace

extern "C" {

gla_status gla_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const void* do_,
                         const void* chunk_states, const float* seg_in, void* dq, void* dk_, void* dv_, float* dg,
                         float* seg_dstate, int B, int H, int T, int dk, int dv, int chunk, int P, int dtype,
                         void* workspace, size_t workspace_size, void* stream) {
  return chunk_bwd_run(q, k, v, g, do_, chunk_states, seg_in, nullptr, dq, dk_, dv_, dg, seg_dstate, B, H, T, dk, dv,
                       chunk, P, dtype, workspace, workspace_size, stream);
}

gla_status gla_chunk_state(const void* k, const void* v, const float* g, float* seg_state, float* seg_logdecay, int B,
                           int H, int T, int dk, int dv, int chunk, int P, int dtype, void* workspace,
                           size_t workspace_size, void* stream) {
  return state_pass_run(GLA_FWD, nullptr, k, v, g, nullptr, seg_state, seg_logdecay, B, H, T, dk, dv, chunk, P, dtype,
                        workspace, workspace_size, stream);
}

gla_status gla_chunk_dstate(const void* q, const float* g, const void* do_, float* seg_dstate, int B, int H, int T,
                            int dk, int dv, int chunk, int P, int dtype, void* workspace, size_t workspace_size,
                            void* stream) {
  return state_pass_run(GLA_BWD, q, nullptr, nullptr, g, do_, seg_dstate, nullptr, B, H, T, dk, dv, chunk, P, dtype,
                        workspace, workspace_size, stream);
}

gla_status gla_chunk_bwd_from(const void* q, const void* k, const void* v, const float* g, const void* do_,
                              const void* chunk_states, const float* seg_in, const float* seg_grad, void* dq,
                              void* dk_, void* dv_, float* dg, int B, int H, int T, int dk, int dv, int chunk, int P,
                              int dtype, void* workspace, size_t workspace_size, void* stream) {
  if (!seg_grad) return fail(GLA_ERR_INVALID_ARG, "gla_chunk_bwd_from: seg_grad must be non-null");
  return chunk_bwd_run(q, k, v, g, do_, chunk_states, seg_in, seg_grad, dq, dk_, dv_, dg, nullptr, B, H, T, dk, dv,
                       chunk, P, dtype, workspace, workspace_size, stream);
}

}  // extern "C"
