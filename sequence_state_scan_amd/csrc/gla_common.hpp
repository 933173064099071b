// Device-side building blocks shared by the GLA kernels (gfx950 / CDNA4, wave64).
//
// Matrix products use the 16x16 MFMA family on 64-lane waves.  For a 16x16 output tile the
// lane l (n16 = l % 16, g4 = l / 16) supplies
//   A operand: A[m = n16][KPL consecutive k-slots owned by group g4]
//   B operand: B[k-slots of group g4][n = n16]
// and receives C[m = 4*g4 + i][n = n16], i = 0..3.  bf16 uses v_mfma_f32_16x16x32_bf16
// (KPL = 8, 32 k per instruction), f32 uses v_mfma_f32_16x16x4_f32 (KPL = 1, 4 k).
// Every product here is written as C[m][n] = sum_k X[m][k] * Y[n][k] with X and Y stored
// k-contiguous ("NT" form), so each lane's fragment is one contiguous LDS read.
//
// Which physical k a slot holds only has to agree between A and B, so a state tile kept in
// accumulator registers (lane holds S[4*g4 + i][n16] of each 16x16 block) can feed the A
// operand directly, and the B operand reads the same k from LDS.  In bf16 two such tiles are
// merged first (merge_pair below): the lane's 8 k-slots are then 8 adjacent k, and the B
// fragment is one 16-byte read.  fp32 takes the slots {16*kb + 4*g4 + i} (mma_regX).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace gla {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves per workgroup
// Leading dimension (elements) of a bf16 LDS tile with rows of D elements (D a multiple of 32).
// Measured on gfx950 with the LDS bank-conflict counter, for a wave whose lane (n16, g4) touches
// row n16 at column 8*g4 (16 bytes) or 4*g4 (8 bytes); conflict cycles per instruction:
//   pad (mod 64)      16-B read   8-B read   16-B write   8-B write   transposing read
//   8, 24, 40              4          0           0            4             2
//   16, 48                 0          2           8           12             2
// and 32 or 0 is worst.  lds_ld pads by 8: tiles written in 16-byte rows and read in 8-byte rows
// or transposed.  lds_ld_frag pads by 16: tiles read mostly as 16-byte MFMA row fragments.
template <typename E>
__host__ __device__ constexpr int lds_ld(int D) { return D + 8; }
template <typename E>
__host__ __device__ constexpr int lds_ld_frag(int D) { return D + 16; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
// threadIdx.x hidden from loop-invariant code motion: the per-lane addresses a long loop body
// derives from it are then recomputed where they are used, not held (or spilled) across the loop.
__device__ __forceinline__ int fresh_tid() {
  int x = threadIdx.x;
  asm volatile("" : "+v"(x));
  return x;
}

// Where a workgroup's tokens lie.  Workgroup i < n_plain is unit i: sub-segment i % S of segment
// i / S, its arrays (init, sub_state, sub_ld) at index i.  With a.list = {n, X, u_0 .. u_{n-1}}
// (written by the state pass over the pieces, resplit_derive),
// workgroup n_plain + j serves piece j % X of unit u_{j / X} (j / X < n): that unit's tokens cut
// into X equal pieces, i.e. sub-segment (u % S) X + j % X of its segment cut into S X, its arrays
// (r_init, r_state, r_ld) at slot j.  With X = 1 the piece is the whole unit, entered from init[u].
struct UnitPlace {
  bool live;
  int unit, seg, sub, NS, X;  // X = 0 for a plain unit
  const float* init;          // the state (gradient) entering the sub-segment from its segment, or null
  float *st, *ld;             // the state pass's outputs
  const float* ldb;           // the summed log-gates of the segment's parts, nld of them, DK apart
  int nld;
};
// Piece j % X of unit `unit`, the listed unit of entry j / X (see unit_place).
template <class A>
__device__ __forceinline__ UnitPlace list_place(const A& a, int j, int X, int unit, int DK, long SS) {
  UnitPlace u{};
  const int x = j % X;
  u.live = true;
  u.unit = unit;
  u.seg = unit / a.S;
  u.sub = (unit - u.seg * a.S) * X + x;
  u.NS = a.S * X;
  u.X = X;
  u.init = X > 1 ? a.r_init + (long)j * SS : a.init ? a.init + (long)unit * SS : nullptr;
  u.st = a.r_state + (long)j * SS;
  u.ld = a.r_ld + (long)j * DK;
  // the segment's log decay: from the unit split's parts where there is one (a unit's is exact at
  // any decay), else from this unit's pieces
  u.ldb = a.S > 1 ? a.sub_ld + (long)u.seg * a.S * DK : a.r_ld + (long)(j - x) * DK;
  u.nld = a.S > 1 ? a.S : X;
  return u;
}
template <class A>
__device__ __forceinline__ UnitPlace unit_place(const A& a, int n_plain, int DK, long SS) {
  const int i = blockIdx.x;
  UnitPlace u{};
  if (i < n_plain) {
    u.live = true;
    u.unit = i;
    u.seg = i / a.S;
    u.sub = i - u.seg * a.S;
    u.NS = a.S;
    u.init = a.init ? a.init + (long)i * SS : nullptr;
    u.st = a.sub_state ? a.sub_state + (long)i * SS : nullptr;
    u.ld = a.sub_ld ? a.sub_ld + (long)i * DK : nullptr;
    u.ldb = a.sub_ld ? a.sub_ld + (long)u.seg * a.S * DK : nullptr;
    u.nld = a.S;
    return u;
  }
  if (!a.list) return u;
  const int j = i - n_plain, n = a.list[0], X = a.list[1], e = j / X;
  if (e >= n) return u;
  return list_place(a, j, X, a.list[2 + e], DK, SS);
}

// The re-split's list, derived from the flags of n_units units by every workgroup of the state pass
// over the pieces (each gets the same): n = min(flagged, R) listed units, the first flagged ones in
// unit order; X = the largest power of 2 <= xmax with n X <= R.  Returns the unit of entry
// slot / X (-1 if slot / X >= n) and sets n and X.  With list non-null it also writes
// list = {n, X, u_0 .. u_{n-1}}.  Every thread of the workgroup calls it (it synchronises the
// workgroup); red: NT / 64 ints of LDS.
template <int NT>
__device__ int resplit_derive(const int* __restrict__ flags, int n_units, int R, int xmax, int slot, int* list, int* red,
                              int& n_out, int& X_out) {
  constexpr int NWV = NT / 64;
  const int lane = lane_id(), wv = threadIdx.x >> 6;
  int c = 0;
  for (int u = threadIdx.x; u < n_units; u += NT) c += flags[u] != 0;
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if (lane == 0) red[wv] = c;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < NWV; ++w) total += red[w];
  __syncthreads();
  const int n = min(total, R);
  int X = xmax;
  while (X > 1 && n * X > R) X >>= 1;
  const int want = slot / X;
  // each flagged unit's rank: the flagged units of the blocks of NT before its own, of the waves
  // before its own, and of the lanes before it
  int found = -1, base = 0;
  for (int u0 = 0; u0 < n_units && base < n; u0 += NT) {
    const int u = u0 + threadIdx.x;
    const bool f = u < n_units && flags[u] != 0;
    const unsigned long long m = __ballot(f);
    if (lane == 0) red[wv] = __popcll(m);
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < NWV; ++w) {
      before += w < wv ? red[w] : 0;
      tot += red[w];
    }
    __syncthreads();
    const int rank = base + before + __popcll(m & ((1ull << lane) - 1ull));
    if (f && rank < n) {
      if (list) list[2 + rank] = u;
      if (rank == want) found = u;
    }
    base += tot;
  }
  if (threadIdx.x == 0) red[0] = -1;
  __syncthreads();
  if (found >= 0) red[0] = found;
  __syncthreads();
  const int unit = red[0];
  __syncthreads();
  if (list && threadIdx.x == 0) {
    list[0] = n;
    list[1] = X;
  }
  n_out = n;
  X_out = X;
  return want < n ? unit : -1;
}

// --------------------------------------------------------------------------------------------
// Element loads and stores (4 or 8 consecutive elements <-> float registers)
// --------------------------------------------------------------------------------------------
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (bf16)x[e];
  *reinterpret_cast<bf16x8*>(p) = a;
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
  f32x4 r;
  r[0] = (float)a[0]; r[1] = (float)a[1]; r[2] = (float)a[2]; r[3] = (float)a[3];
  return r;
}
__device__ __forceinline__ void store4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ void store4(bf16* p, f32x4 x) {
  bf16x4 a;
  a[0] = (bf16)x[0]; a[1] = (bf16)x[1]; a[2] = (bf16)x[2]; a[3] = (bf16)x[3];
  *reinterpret_cast<bf16x4*>(p) = a;
}

// Streaming (nontemporal) global accesses.  Used only where one wave instruction covers whole
// 128-byte lines: the rows of V and dO, and the chunk-state tiles (512 or 1024 contiguous
// bytes).  There the streaming policy raised throughput by a few percent on gfx950.  Accesses
// that cover half a line per instruction (gate tiles, merged output pairs) were much slower with
// it, presumably because the line is dropped before the other half arrives, so they keep the
// default policy.
template <typename T>
__device__ __forceinline__ T gld_nt(const T* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void gst_nt(float* p, f32x4 x) { __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p)); }
__device__ __forceinline__ void gst_nt(bf16* p, f32x4 x) {
  bf16x4 a;
  a[0] = (bf16)x[0]; a[1] = (bf16)x[1]; a[2] = (bf16)x[2]; a[3] = (bf16)x[3];
  __builtin_nontemporal_store(a, reinterpret_cast<bf16x4*>(p));
}

// --------------------------------------------------------------------------------------------
// MFMA
// --------------------------------------------------------------------------------------------
template <typename E> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int KSTEP = 32, KPL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static frag ld(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int KSTEP = 4, KPL = 1;
  typedef float frag;
  __device__ __forceinline__ static frag ld(const float* p) { return *p; }
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x4 zero4() { f32x4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Fragment of an operand Z[m][k] for the 16 rows m0..m0+15 at k-step kk, read from LDS.
//   TR == false: Z stored k-contiguous, row m at P + m * ld (P points at row m0).
//   TR == true:  Z stored transposed, ZT[k][m] at P + k * ld + m (P points at column m0).
// bf16 TR uses ds_read_b64_tr_b16: in each 16-lane group, lane i receives element (i % 4) of
// the 8-byte chunks addressed by lanes 4e + i/4 (e = 0..3).  Lane s of group g4 therefore
// addresses ZT[kk + 8*g4 + s/4 (+4)][4*(s%4)] and receives Z[m0 + s][kk + 8*g4 + 0..3 (4..7)].
template <typename E, bool TR>
__device__ __forceinline__ typename Mma<E>::frag frag_ld(const E* P, int ld, int kk) {
  const int l = lane_id(), s = l & 15, g4 = l >> 4;
  if constexpr (sizeof(E) == 2) {
    if constexpr (!TR) {
      return *reinterpret_cast<const bf16x8*>(P + s * ld + kk + 8 * g4);
    } else {
      typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lbf16x4;
      const E* p0 = P + (kk + 8 * g4 + (s >> 2)) * ld + 4 * (s & 3);
      const lbf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) lbf16x4*)(p0));
      const lbf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) lbf16x4*)(p0 + 4 * ld));
      bf16x8 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) { r[e] = lo[e]; r[4 + e] = hi[e]; }
      return r;
    }
  } else {
    if constexpr (!TR) return P[s * ld + kk + g4];
    else return P[(kk + g4) * ld + s];
  }
}

// acc[m][n] += sum_{k in [kb, ke)} X[m][k] Y[n][k]; XTR / YTR select the storage of X and Y
// as in frag_ld.  kb, ke multiples of Mma<E>::KSTEP.
template <typename E, bool XTR, bool YTR>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const E* X, int ldx, const E* Y, int ldy, int kb, int ke) {
#pragma unroll 4
  for (int kk = kb; kk < ke; kk += Mma<E>::KSTEP)
    acc = Mma<E>::mma(frag_ld<E, XTR>(X, ldx, kk), frag_ld<E, YTR>(Y, ldy, kk), acc);
  return acc;
}

// fp32: acc[m][n] += sum_k X[m][k] * Y[n][k] where X comes from NKB accumulator-layout register
// tiles: R[kb][i] holds X[m = n16][k = 16*kb + 4*g4 + i].  Yrow points at Y's row n = n16 of this
// tile (so the lane reads Y[n16][16*kb + 4*g4 + i]).  (bf16 callers merge pairs of tiles with
// merge_pair instead, so that their Y fragment is one 16-byte read.)
template <int NKB>
__device__ __forceinline__ f32x4 mma_regX(f32x4 acc, const f32x4 (&R)[NKB], const float* Yrow) {
  const int g4 = lane_id() >> 4;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = Mma<float>::mma(R[kb][i], Yrow[16 * kb + 4 * g4 + i], acc);
  return acc;
}

// fp32: acc[tT] += X . Y_tT^T for NTT row blocks of Y at once, X from accumulator registers as in
// mma_regX; the lane's Y row for block tT is Y0 + tT * ldblk.
template <int NKB, int NTT>
__device__ __forceinline__ void mma_regX_rows(f32x4 (&acc)[NTT], const f32x4 (&R)[NKB], const float* Y0, int ldblk) {
  const int g4 = lane_id() >> 4;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tT = 0; tT < NTT; ++tT) acc[tT] = Mma<float>::mma(R[kb][i], (Y0 + tT * ldblk)[16 * kb + 4 * g4 + i], acc[tT]);
}

// Same as mma_regX, with X given as pieces already in the element type: R[kb] holds
// X[m = n16][k = 16*kb + 4*g4 + 0..3] (bf16x4 for bf16, f32x4 for float).
template <typename E> struct Piece4 { typedef f32x4 type; };
template <> struct Piece4<bf16> { typedef bf16x4 type; };

template <typename E>
__device__ __forceinline__ typename Piece4<E>::type load_piece(const E* p) {
  return *reinterpret_cast<const typename Piece4<E>::type*>(p);
}
__device__ __forceinline__ f32x4 widen(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 widen(bf16x4 x) {
  f32x4 r;
  r[0] = (float)x[0]; r[1] = (float)x[1]; r[2] = (float)x[2]; r[3] = (float)x[3];
  return r;
}

template <typename E, int NKB>
__device__ __forceinline__ f32x4 mma_regX_e(f32x4 acc, const typename Piece4<E>::type (&R)[NKB], const E* Yrow) {
  const int g4 = lane_id() >> 4;
  if constexpr (sizeof(E) == 2) {
    static_assert(NKB % 2 == 0, "bf16 pieces come in pairs");
#pragma unroll
    for (int p = 0; p < NKB / 2; ++p) {
      bf16x8 x, y;
      const bf16x4 ylo = *reinterpret_cast<const bf16x4*>(Yrow + 32 * p + 4 * g4);
      const bf16x4 yhi = *reinterpret_cast<const bf16x4*>(Yrow + 32 * p + 16 + 4 * g4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = R[2 * p][i];
        x[4 + i] = R[2 * p + 1][i];
        y[i] = ylo[i];
        y[4 + i] = yhi[i];
      }
      acc = Mma<bf16>::mma(x, y, acc);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = Mma<float>::mma(R[kb][i], Yrow[16 * kb + 4 * g4 + i], acc);
  }
  return acc;
}

__device__ __forceinline__ float piece_dot(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }
// bf16 pieces on both sides: two v_dot2_f32_bf16 (bf16 products are exact in fp32, summed in fp32).
__device__ __forceinline__ float piece_dot(bf16x4 a, bf16x4 b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 alo = {a[0], a[1]}, ahi = {a[2], a[3]}, blo = {b[0], b[1]}, bhi = {b[2], b[3]};
  return __builtin_amdgcn_fdot2_f32_bf16(ahi, bhi, __builtin_amdgcn_fdot2_f32_bf16(alo, blo, 0.f, false), false);
}
__device__ __forceinline__ float piece_dot(bf16x4 a, f32x4 b) {
  return (float)a[0] * b[0] + (float)a[1] * b[1] + (float)a[2] * b[2] + (float)a[3] * b[3];
}

// Sum over the four lanes that share n16 (lanes n16, n16+16, n16+32, n16+48).
__device__ __forceinline__ float sum_over_g4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// --------------------------------------------------------------------------------------------
// 4x4 transpose inside each quad of lanes (lanes 4m..4m+3), with DPP quad permutes.  On entry
// lane 4m+r holds column r of a 4x4 block (x[i] = M[i][r]); on exit it holds row r
// (x[c] = M[r][c]).  Used to turn an accumulator tile (4 consecutive rows per lane) into
// 4 consecutive columns per lane for 8-byte stores.
// --------------------------------------------------------------------------------------------
__device__ __forceinline__ float dpp_quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
}
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x) {
  const int r = lane_id() & 3;
  const bool hi2 = r & 2, hi1 = r & 1;
  // exchange the off-diagonal 2x2 blocks with lane r^2
  float s0 = hi2 ? x[0] : x[2], s1 = hi2 ? x[1] : x[3];
  float r0 = dpp_quad_xor2(s0), r1 = dpp_quad_xor2(s1);
  if (hi2) { x[0] = r0; x[1] = r1; } else { x[2] = r0; x[3] = r1; }
  // exchange inside each 2x2 block with lane r^1
  s0 = hi1 ? x[0] : x[1];
  s1 = hi1 ? x[2] : x[3];
  r0 = dpp_quad_xor1(s0);
  r1 = dpp_quad_xor1(s1);
  if (hi1) { x[0] = r0; x[2] = r1; } else { x[1] = r0; x[3] = r1; }
  return x;
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
  return r;
}
__device__ __forceinline__ bf16x8 join_bf16x4(bf16x4 x, bf16x4 y) {
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// --------------------------------------------------------------------------------------------
// Chunk-state tiles.  A dk x dv chunk state is stored as (dk/16) x (dv/16) tiles of 16 x 16
// elements.  Element (r, q) of a tile belongs to lane index L = 16 (q / 4) + r, position q % 4.
// With dv/16 even, tiles (cb, 2m) and (cb, 2m + 1) are interleaved: lane index L of the pair holds
// 8 consecutive elements, its 4 of tile 2m and then its 4 of tile 2m + 1, at element offset
// (cb * dv/16 + 2m) * 256 + 8 L.  With dv/16 odd (only dv = 16) tile (cb, jb) holds its 4 at
// (cb * dv/16 + jb) * 256 + 4 L.  A wave whose lanes hold both tiles of a pair in one of the lane
// layouts below moves them with one 16-byte access per lane (bf16): 1024 contiguous bytes.
// --------------------------------------------------------------------------------------------
template <int NJB>
__device__ __forceinline__ long state_at(int cb, int jb, int L) {
  if constexpr (NJB % 2 == 0) return (long)(cb * NJB + (jb & ~1)) * 256 + 8 * L + 4 * (jb & 1);
  else return (long)(cb * NJB + jb) * 256 + 4 * L;
}
// lane index of lane (n16, g4) holding row n16, columns 4g4..4g4+3 of a tile
__device__ __forceinline__ int state_lane_row(int n16, int g4) { return 16 * g4 + n16; }
// lane index of lane (n16, g4) holding an accumulator tile X[4g4 + i][n16] after quad_transpose:
// row 4g4 + (n16 & 3), columns (n16 & ~3) + i
__device__ __forceinline__ int state_lane_qt(int n16, int g4) { return 16 * (n16 >> 2) + 4 * g4 + (n16 & 3); }

// The lane's pieces of tiles (cb, 2m) and (cb, 2m + 1) (streaming loads; dv/16 even)
template <typename E, int NJB>
__device__ __forceinline__ void load_state_pair(const E* st, int cb, int m, int L, typename Piece4<E>::type& a,
                                                typename Piece4<E>::type& b) {
  typedef typename Piece4<E>::type piece;
  static_assert(NJB % 2 == 0, "tiles pair up along dv");
  if constexpr (sizeof(E) == 2) {
    const bf16x8 x = gld_nt(reinterpret_cast<const bf16x8*>(st + state_at<NJB>(cb, 2 * m, L)));
    a = __builtin_shufflevector(x, x, 0, 1, 2, 3);
    b = __builtin_shufflevector(x, x, 4, 5, 6, 7);
  } else {
    a = gld_nt(reinterpret_cast<const piece*>(st + state_at<NJB>(cb, 2 * m, L)));
    b = gld_nt(reinterpret_cast<const piece*>(st + state_at<NJB>(cb, 2 * m + 1, L)));
  }
}
template <typename E, int NJB>
__device__ __forceinline__ typename Piece4<E>::type load_state_piece(const E* st, int cb, int jb, int L) {
  return gld_nt(reinterpret_cast<const typename Piece4<E>::type*>(st + state_at<NJB>(cb, jb, L)));
}
template <typename E, int NJB>
__device__ __forceinline__ void store_state_pair(E* st, int cb, int m, int L, f32x4 a, f32x4 b) {
  static_assert(NJB % 2 == 0, "tiles pair up along dv");
  if constexpr (sizeof(E) == 2) {
    __builtin_nontemporal_store(join_bf16x4(to_bf16x4(a), to_bf16x4(b)),
                                reinterpret_cast<bf16x8*>(st + state_at<NJB>(cb, 2 * m, L)));
  } else {
    gst_nt(st + state_at<NJB>(cb, 2 * m, L), a);
    gst_nt(st + state_at<NJB>(cb, 2 * m + 1, L), b);
  }
}
template <typename E, int NJB>
__device__ __forceinline__ void store_state_piece(E* st, int cb, int jb, int L, f32x4 a) {
  gst_nt(st + state_at<NJB>(cb, jb, L), a);
}

// --------------------------------------------------------------------------------------------
// Wider stores of two adjacent 16-column blocks.  X and Y hold, in lane (n16, g4), row n16 and
// columns 4g4..4g4+3 of the left and the right block.  v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second: swapping the packed pairs of X and Y
// leaves lane rows 0 and 2 with 8 consecutive columns of X (0..7, 8..15) and rows 1 and 3 with
// those of Y.  Each lane then stores 16 bytes at column pair_col(g4) of the 32-column pair, the
// four lane rows covering 64 contiguous bytes of each row.
// --------------------------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 merge_pair(bf16x4 X, bf16x4 Y) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x2 xd = __builtin_bit_cast(u32x2, X), yd = __builtin_bit_cast(u32x2, Y);
  const auto s0 = __builtin_amdgcn_permlane16_swap(xd[0], yd[0], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(xd[1], yd[1], false, false);
  const u32x4 r = {s0[0], s1[0], s0[1], s1[1]};
  return __builtin_bit_cast(bf16x8, r);
}
__device__ __forceinline__ int pair_col(int g4) { return 8 * (g4 >> 1) + 16 * (g4 & 1); }
// The inverse, for a read-modify-write: the swap is its own inverse, so a piece loaded from
// column pair_col(g4) gives back X and Y in the accumulator layout.
__device__ __forceinline__ void unmerge_pair(bf16x8 m, bf16x4& X, bf16x4& Y) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 d = __builtin_bit_cast(u32x4, m);
  const auto s0 = __builtin_amdgcn_permlane16_swap(d[0], d[2], false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(d[1], d[3], false, false);
  const u32x2 x = {s0[0], s1[0]}, y = {s0[1], s1[1]};
  X = __builtin_bit_cast(bf16x4, x);
  Y = __builtin_bit_cast(bf16x4, y);
}

// --------------------------------------------------------------------------------------------
// Segmented scans across lanes: segments of W consecutive lanes (W a power of two, W <= 16), on
// DPP row shifts inside the 16-lane rows (a lane whose source lies outside its row reads 0).
// --------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_zero_fill(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Sum of x over the 16 lanes of the DPP row, on every lane of the row (rotations by 8, 4, 2, 1).
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, false));  // row_ror:1
  return x;
}
template <int D> __device__ __forceinline__ float row_shr(float x) { return dpp_zero_fill<0x110 + D>(x); }
template <int D> __device__ __forceinline__ float row_shl(float x) { return dpp_zero_fill<0x100 + D>(x); }

// Inclusive prefix sum of x over the lanes of the segment (lane order).
template <int W>
__device__ __forceinline__ float seg_scan_incl(float x) {
  static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "segments of 1, 2, 4, 8 or 16 lanes");
  const int i = lane_id() & (W - 1);
  if constexpr (W > 1) { const float y = row_shr<1>(x); x += (W == 16 || i >= 1) ? y : 0.f; }
  if constexpr (W > 2) { const float y = row_shr<2>(x); x += (W == 16 || i >= 2) ? y : 0.f; }
  if constexpr (W > 4) { const float y = row_shr<4>(x); x += (W == 16 || i >= 4) ? y : 0.f; }
  if constexpr (W > 8) x += row_shr<8>(x);
  return x;
}
// Inclusive suffix sum of x over the lanes of the segment (from the segment's last lane down).
template <int W>
__device__ __forceinline__ float seg_scan_rev_incl(float x) {
  static_assert(W >= 1 && W <= 16 && (W & (W - 1)) == 0, "segments of 1, 2, 4, 8 or 16 lanes");
  const int i = lane_id() & (W - 1);
  if constexpr (W > 1) { const float y = row_shl<1>(x); x += (W == 16 || i + 1 < W) ? y : 0.f; }
  if constexpr (W > 2) { const float y = row_shl<2>(x); x += (W == 16 || i + 2 < W) ? y : 0.f; }
  if constexpr (W > 4) { const float y = row_shl<4>(x); x += (W == 16 || i + 4 < W) ? y : 0.f; }
  if constexpr (W > 8) x += row_shl<8>(x);
  return x;
}
// Value of x at the segment's last lane, on every lane of the segment.
template <int W>
__device__ __forceinline__ float seg_last(float x) {
  if constexpr (W == 16)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xF, 0xF, false));  // row_newbcast:15
  else
    return __shfl(x, W - 1, W);
}

// R rows of 4 consecutive elements of a row-major tensor (rows ld apart), held in registers for
// prefetching.  With ld = 16 rows of the tensor this is a "strided item": lane n16 of a 16-lane row
// holds tokens n16, n16 + 16, ... of a chunk, so the 16 lanes of a row cover 16 consecutive tokens.
template <typename E, int R> struct RowsRx4;
template <int R> struct RowsRx4<bf16, R> {
  bf16x4 r[R];
  __device__ __forceinline__ void load(const bf16* p, long ld) {
#pragma unroll
    for (int i = 0; i < R; ++i) r[i] = *reinterpret_cast<const bf16x4*>(p + i * ld);
  }
  __device__ __forceinline__ float at(int i, int e) const { return (float)r[i][e]; }
};
template <int R> struct RowsRx4<float, R> {
  f32x4 r[R];
  __device__ __forceinline__ void load(const float* p, long ld) {
#pragma unroll
    for (int i = 0; i < R; ++i) r[i] = *reinterpret_cast<const f32x4*>(p + i * ld);
  }
  __device__ __forceinline__ float at(int i, int e) const { return r[i][e]; }
};

// Gate prefix sums of a strided item (tokens 16i + n16 of the chunk, i < R; 4 channels), the 16
// lanes of a row holding 16 consecutive tokens: on return b[i][e] is the in-chunk inclusive running
// sum of g at token 16i + n16 and lam[e] the chunk total.  One DPP row scan per 16-token block.
template <int R, class Rows>
__device__ __forceinline__ void chunk_gate_prefix_strided(const Rows& pg, bool has_item, float (&b)[R][4],
                                                          float (&lam)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float run = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float incl = seg_scan_incl<16>(has_item ? pg.at(i, e) : 0.f);
      b[i][e] = run + incl;
      run += seg_last<16>(incl);
    }
    lam[e] = run;
  }
}

// 8 consecutive elements of a row in registers: one 16-byte piece for bf16, two for float.
template <typename E> struct Piece8;
template <> struct Piece8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ float at(int e) const { return (float)v[e]; }
};
template <> struct Piece8<float> {
  f32x4 lo, hi;
  __device__ __forceinline__ void load(const float* p) {
    lo = load4(p);
    hi = load4(p + 4);
  }
  __device__ __forceinline__ float at(int e) const { return e < 4 ? lo[e] : hi[e - 4]; }
};

// Gate tile of a chunk in items of 16 tokens x 8 channels.  Lane row R = tid / 16 takes channel
// group x = R % (DK / 8), channels 8x..8x+7, and the RI token blocks set*RI.. with set =
// R / (DK / 8); lane n16 of the row holds token 16 * block + n16 of each.  So a load of q or k
// reads 16 bytes per lane and the 4 lane rows of a wave cover 64 contiguous bytes of each of 16
// token rows; a load of g reads 4 channels per lane and the pair of loads covers 128 contiguous
// bytes per token row.  The 16 lanes of a row hold 16 consecutive tokens, so the in-block
// running sums are DPP row scans; the NSET sets of token blocks meet through LDS.
template <typename E, int C, int DK, int NT>
struct GateTile8 {
  static constexpr int NCG = DK / 8, NTB = C / 16, NROW = NT / 16;
  static constexpr int RI = NTB * NCG >= NROW ? NTB * NCG / NROW : 1;  // token blocks per lane row
  static constexpr int NSET = NTB / RI;                                 // lane rows per channel group
  static constexpr int NACT = 16 * NCG * NSET;                          // threads holding an item
  static_assert(NTB % RI == 0 && NACT <= NT, "items of 16 tokens x 8 channels tile the chunk");
  f32x4 g[RI][2];
  Piece8<E> q[RI], k[RI];

  static __device__ __forceinline__ bool active(int tid) { return NACT == NT || tid < NACT; }
  static __device__ __forceinline__ int set_of(int tid) { return (tid >> 4) / NCG; }
  static __device__ __forceinline__ int group_of(int tid) { return (tid >> 4) % NCG; }
  // chunk row (token) of block r of the thread's item
  static __device__ __forceinline__ int row(int tid, int r) { return 16 * (set_of(tid) * RI + r) + (tid & 15); }

  // chunk_elem: element offset of the chunk's first token (token index * DK); qp or kp may be
  // null (then q or k is not loaded)
  __device__ __forceinline__ void load(const float* gp, const E* qp, const E* kp, long chunk_elem, int tid) {
    if (!active(tid)) return;
    const long off = chunk_elem + (long)row(tid, 0) * DK + 8 * group_of(tid);
#pragma unroll
    for (int r = 0; r < RI; ++r) {
      g[r][0] = load4(gp + off + r * 16 * DK);
      g[r][1] = load4(gp + off + r * 16 * DK + 4);
      if (qp) q[r].load(qp + off + r * 16 * DK);
      if (kp) k[r].load(kp + off + r * 16 * DK);
    }
  }
  __device__ __forceinline__ float gat(int r, int e) const { return g[r][e >> 2][e & 3]; }

  // b[r][e]: in-chunk inclusive running sum of g at the thread's token of block r, channel 8x + e;
  // lam[e]: the chunk total of that channel.  sTot: NSET * DK floats of LDS.  With NSET > 1 this
  // holds a barrier: every thread of the workgroup calls it.
  __device__ __forceinline__ void prefix(int tid, float* sTot, float (&b)[RI][8], float (&lam)[8]) const {
    const bool act = active(tid);
    float run[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      run[e] = 0.f;
#pragma unroll
      for (int r = 0; r < RI; ++r) {
        const float incl = seg_scan_incl<16>(act ? gat(r, e) : 0.f);
        b[r][e] = run[e] + incl;
        run[e] += seg_last<16>(incl);
      }
      lam[e] = run[e];
    }
    if constexpr (NSET > 1) {
      const int set = set_of(tid), x = group_of(tid);
      if (act && (tid & 15) == 0) {
        store4(sTot + set * DK + 8 * x, f32x4{run[0], run[1], run[2], run[3]});
        store4(sTot + set * DK + 8 * x + 4, f32x4{run[4], run[5], run[6], run[7]});
      }
      __syncthreads();
      if (act) {
        float before[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) before[e] = lam[e] = 0.f;
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
          const f32x4 lo = load4(sTot + s * DK + 8 * x), hi = load4(sTot + s * DK + 8 * x + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float t = e < 4 ? lo[e] : hi[e - 4];
            lam[e] += t;
            if (s < set) before[e] += t;
          }
        }
#pragma unroll
        for (int r = 0; r < RI; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) b[r][e] += before[e];
      }
    }
  }
};

// 8 consecutive elements (16 bytes for bf16, 32 for float) copied global -> registers -> LDS.
template <typename E> struct Vec8;
template <> struct Vec8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = gld_nt(reinterpret_cast<const bf16x8*>(p)); }
  __device__ __forceinline__ void store(bf16* p) const { *reinterpret_cast<bf16x8*>(p) = v; }
};
template <> struct Vec8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = load4(p);
    b = load4(p + 4);
  }
  __device__ __forceinline__ void store(float* p) const {
    store4(p, a);
    store4(p + 4, b);
  }
};

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// --------------------------------------------------------------------------------------------
// Exactness of the chunk factorisation.  The fast kernels factor exp(b_t - b_s) inside a chunk as
// exp(b_t) * exp(-b_s) (K/Lambda).  They handle a chunk only when every channel's chunk decay is
// at least kFastMinChunkLogDecay: exp(-b) then stays below exp(40) ~ 2.4e17 and exp(b) above
// 4e-18, far from the float32 and bfloat16 limits.  A unit (b, h, segment) with any stronger chunk
// is recorded in the per-unit flags and recomputed by the exact sub-block kernels.
// --------------------------------------------------------------------------------------------
constexpr float kFastMinChunkLogDecay = -40.f;

// The reach of a segment's decay.  A token's share of a segment's end state (or of the gradient
// entering it) carries the factor exp(x), x the summed log-gates between the token and the
// segment's far end.  Below x = kReachCut both exp and __expf give exactly 0.0f in float32
// (e^-112 ~ 2e-49, under the smallest subnormal), and with g <= 0 x only falls further along the
// walk, so a state pass that walks from the far end may stop once every channel is past it: the
// chunks it leaves out contribute exact zeros.
constexpr float kReachCut = -112.f;

// A workgroup-uniform OR of pred at a barrier: every wave writes its ballot to its slot of sLive
// ([2][NW] ints, the half picked by parity), the barrier follows, and every lane reads the NW
// slots.  Loops calling it once per iteration alternate parity: a slot is written again only two
// barriers after it was read.
template <int NW>
__device__ __forceinline__ bool barrier_any(int* sLive, int parity, bool pred) {
  const int wave = __ballot(pred) != 0;
  if (lane_id() == 0) sLive[parity * NW + wave_id()] = wave;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) any |= sLive[parity * NW + i];
  return any != 0;
}

// Broadcast lane S of each 16-lane row to the whole row (DPP row_newbcast).
template <int S>
__device__ __forceinline__ float row_bcast(float x) {
  static_assert(S >= 0 && S < 16, "a lane of the row");
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + S, 0xF, 0xF, false));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// acc[m][n] += sum_{k < 16} X[m][k] Y[n][k] (a contraction over one 16-token sub-block), with XTR /
// YTR selecting the storage of X and Y as in frag_ld.  bf16 runs v_mfma_f32_16x16x32_bf16 with the
// upper 16 k-slots zero: lanes g4 = 0, 1 supply k = 8 g4 .. 8 g4 + 7, lanes g4 = 2, 3 zeros (their
// reads are pointed back at rows g4 - 2, inside the tile, and discarded).  The 16-deep
// v_mfma_f32_16x16x16_bf16 is not used: when its result fed the next MFMA as the accumulator, the
// upper two result registers read back stale now and then on gfx950.  f32 takes four
// v_mfma_f32_16x16x4_f32.
template <typename E, bool XTR, bool YTR>
__device__ __forceinline__ f32x4 mma_k16(f32x4 acc, const E* X, int ldx, const E* Y, int ldy) {
  if constexpr (sizeof(E) == 2) {
    const int g4 = lane_id() >> 4, kk = -16 * (g4 >> 1);
    bf16x8 x = frag_ld<E, XTR>(X, ldx, kk), y = frag_ld<E, YTR>(Y, ldy, kk);
    if (g4 >= 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = y[e] = (E)0.f;
    }
    return Mma<bf16>::mma(x, y, acc);
  } else {
    return mma<E, XTR, YTR>(acc, X, ldx, Y, ldy, 0, 16);
  }
}

}  // namespace gla
