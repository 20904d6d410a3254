// kernels.hip -- gfx950 kernels: the fused-group op-program executor, the
// tensor-fusion bucket pack/unpack kernel and a plain copy kernel.
//
// Executor.  One launch runs one fused group (TVM "Operator Fusion":
// FuseOps forms the group, FuseTIR merges it into one function whose
// intermediates never touch device memory; DisCo section 1: op fusion
// saves the intermediate traffic and the launches).  Each workgroup takes
// items = (row block, column panel) in a grid-stride loop:
//   1. column phase: every thread runs the column program for some columns
//      of the panel; results ([1,C] broadcast operands) go to LDS once per
//      workgroup (once per item when a row spans several panels);
//   2. row phase: one thread per row of the block runs the row program
//      ([R,1] operands such as a LayerNorm's mean and 1/std) into LDS;
//   3. element phase: threads are split into rows of 1 << tpr_log2 lanes;
//      each lane walks its row in tiles of kV elements, 16-byte loads and
//      stores, and runs the element program with the tile in VGPRs;
//   4. reduce tail (when the group ends in a row reduction): per-lane fp32
//      partial sums, a butterfly over the row's lanes with DPP
//      (quad_perm, row_half_mirror, row_mirror) and wave shuffles, and for
//      rows wider than a wave a cross-wave combine through LDS in a fixed
//      order, so the result is deterministic.
//
// The interpreter dispatches on a wave-uniform instruction word (a scalar
// load from the kernarg segment, fetched one instruction ahead, and a
// scalar branch tree).  Its registers A, B and six spill slots each hold a
// tile; every register index is a compile-time constant of its case, so
// they stay in VGPRs, and each op has a single body.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>

#include "gtf.h"
#include "isa.h"
#include "plan.h"

namespace gtf {

enum Mode { M_ELEM = 0, M_ROW = 1, M_COL = 2 };

// Address spaces made explicit, so that data accesses stay global_load /
// global_store and slot-pointer reads stay scalar loads wherever the
// pointers come from (kernel arguments or a device table).
#define GAS __attribute__((address_space(1)))
#define CAS __attribute__((address_space(4)))
typedef void* const CAS SlotPtr;  // a slot's base pointer, read with s_load
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // fp32 -> bf16 round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
// The same for two values stored side by side, both halves in one
// v_cvt_pk_bf16_f32 (round to nearest even, like the compiler's own
// conversion).  The compiler converts pack_bf16's halves one by one and
// joins them with a shift and an or; written as a two-lane vector
// conversion it does pair them, but then schedules the interpreter's
// store case so that other instances spill.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}

// e^x for x <= 0: 2^(x log2 e) on the hardware base-2 exponential
// (v_exp_f32, about 1 ulp), with x log2 e carried as yh + yl: yh = fl(x L)
// with L = log2 e rounded to fp32, yl = the exact error of that product
// (one fma) plus x times the rest of log2 e.  Then e^x = 2^yh (1 + yl ln 2)
// up to (yl ln 2)^2 / 2 < 1e-10 relative.  About 1.5 ulp in all, against
// about 12 VALU slots for the library expf, which also handles overflow, out
// of reach for a non-positive argument.  Results below the normal range
// come out of v_exp_f32 flushed.
// yl is computed from x clamped to [-104, 0] (one v_med3, no lane mask):
// at -inf, or where x L overflows, the error term of the unclamped product
// would be -inf + inf = NaN, while below -104 e^x rounds to 0 whatever yl
// is.  yh keeps the unclamped x, so -inf gives 0 and NaN stays NaN.
struct ExpSplit {
  float yh, yl;
};
__device__ __forceinline__ ExpSplit exp_split(float x) {
  constexpr float kL = 1.44269502e+00f;       // log2(e) rounded to fp32
  constexpr float kLlo = 1.92596299e-08f;     // log2(e) - kL
  const float xc = __builtin_amdgcn_fmed3f(x, -104.0f, 0.0f);
  const float yc = xc * kL;
  return ExpSplit{x * kL, __builtin_fmaf(xc, kL, -yc) + xc * kLlo};
}
__device__ __forceinline__ float exp_nonpos(float x) {
  constexpr float kLn2 = 6.93147182e-01f;
  const ExpSplit y = exp_split(x);
  const float p = __builtin_amdgcn_exp2f(y.yh);
  return __builtin_fmaf(p, y.yl * kLn2, p);
}
// The same, keeping results in fp32's subnormal range (the tails of sigmoid
// and the fp32 GELU are results in their own right): 2^yh is taken as the
// square of 2^(yh / 2), which is normal down to yh = -252, so the square
// underflows gradually, correctly rounded, instead of being flushed.  Two
// VALU slots more and about one ulp more error.
__device__ __forceinline__ float exp_nonpos_sub(float x) {
  constexpr float kLn2 = 6.93147182e-01f;
  const ExpSplit y = exp_split(x);
  const float h = __builtin_amdgcn_exp2f(y.yh * 0.5f);
  // h (1 + yl ln 2) is normal, so the one rounding into the subnormal range
  // is the last product's
  return __builtin_fmaf(h, y.yl * kLn2, h) * h;
}

// e^x over the whole range: the split of x log2 e as in exp_nonpos (the
// error term from x clamped to [-104, 89], one v_med3), 2^yh as the square
// of 2^(yh / 2) so that results in fp32's subnormal range round gradually
// and results past its top overflow to +inf, and the correction applied as
// a factor 1 + yl ln 2 (as an fma against h, h = +inf would meet a negative
// correction as inf - inf).  About 3 ulp; 9 VALU slots against 13 for the
// library expf.  -inf gives 0, +inf gives +inf, NaN stays NaN.
__device__ __forceinline__ float f_exp(float x) {
  constexpr float kL = 1.44269502e+00f;
  constexpr float kLlo = 1.92596299e-08f;
  constexpr float kLn2 = 6.93147182e-01f;
  const float xc = __builtin_amdgcn_fmed3f(x, -104.0f, 89.0f);
  const float yc = xc * kL;
  const float yl = __builtin_fmaf(xc, kLlo, __builtin_fmaf(xc, kL, -yc));
  const float h = __builtin_amdgcn_exp2f(x * (0.5f * kL));
  // h (1 + yl ln 2) is normal wherever h is, so the one rounding into the
  // subnormal range is the last product's
  return (h * __builtin_fmaf(yl, kLn2, 1.0f)) * h;
}

__device__ __forceinline__ float f_sigmoid(float x) {
  // 1 / (1 + e^-x), written as e^x / (1 + e^x) for x < 0 so the tail keeps
  // its relative accuracy; one correctly rounded division
  const float e = exp_nonpos_sub(-fabsf(x));
  const float num = x >= 0.f ? 1.f : e;
  return num / (1.f + e);
}
// gelu(x) = x * Phi(x), Phi the standard normal CDF (the exact GELU).  With
// t = |x| and Q(t) = P(Z > t) = exp(-t^2/2) * R(t):  Phi(x) = 1 - Q(t) for
// x >= 0 and Q(t) for x < 0, so the negative tail keeps its relative
// accuracy without ever forming 1 + erf.
//  * exp(-t^2/2): t^2 = hi + lo exactly (one fma), then
//    exp(-hi/2) * (1 - lo/2); the argument is never rounded.
//  * R(t) = M(t) / sqrt(2 pi), M the Mills ratio, is u * P8(u) with
//    u = 1 / (1 + p t).  p and P8 were fitted for this kernel by
//    iteratively reweighted least squares toward the minimax relative error
//    on t in [0, 13.5] against the float64 reference 0.5 * erfcx(t/sqrt(2)):
//    fit error 2.0e-8, Horner condition number below 2.4.
// End to end in fp32 (with exp_nonpos and a 1-ulp reciprocal) the relative
// error stays below 1e-6.  t is clamped at 20 for the exponential, where it
// is 0 in fp32, so +inf gives +inf and -inf gives NaN (inf * 0) as the
// definition does.  About 31 VALU slots per element.
constexpr float kGeluP = 3.45e-01f;
__device__ __forceinline__ float f_gelu(float x) {
  const float t = fabsf(x);
  const float tc = fminf(t, 20.0f);
  const float hi = tc * tc;
  const float lo = __builtin_fmaf(tc, tc, -hi);
  float e = exp_nonpos_sub(-0.5f * hi);
  e = __builtin_fmaf(e, -0.5f * lo, e);
  const float u = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluP, t, 1.0f));
  float P = -2.8428646e-02f;
  P = __builtin_fmaf(P, u, 1.4549498e-01f);
  P = __builtin_fmaf(P, u, -2.7158445e-01f);
  P = __builtin_fmaf(P, u, 1.876345e-01f);
  P = __builtin_fmaf(P, u, -3.7881684e-02f);
  P = __builtin_fmaf(P, u, 1.1190944e-01f);
  P = __builtin_fmaf(P, u, 1.1721255e-01f);
  P = __builtin_fmaf(P, u, 1.3802417e-01f);
  P = __builtin_fmaf(P, u, 1.3761912e-01f);
  const float q = e * (u * P);
  const float phi = x >= 0.f ? 1.0f - q : q;
  return x * phi;
}
// The same GELU for a result that is rounded to bf16 and read by nothing
// else.  Half a bf16 ulp is 2^-9 of the value or more, so a relative error
// far below that still rounds to the exact value's bf16 neighbour or to its
// rounding itself.  Q(t) = exp(-t^2/2) u P3(u), u = 1 / (1 + p t), with p and
// the degree-3 P fitted here (Lawson's minimax iteration on the relative
// error over t in [0, 13.7], where the bf16 result is still nonzero,
// against the float64 reference 0.5 erfcx(t / sqrt 2)): 2.3e-4, and about
// the same evaluated in fp32 -- 8x inside the budget.  exp(-t^2/2) is the
// square of h = 2^(-t^2 log2(e) / 4), which stays normal where the square
// is a subnormal, so the square rounds gradually instead of flushing: bf16
// subnormal results (t beyond about 13.2) come out right.  For t = inf or
// t^2 beyond fp32 both h and u are 0, so +inf gives +inf and -inf gives
// NaN (inf * 0), as the definition does.  About 15 VALU slots.
constexpr float kGeluBfP = 4.9930957e-01f;
__device__ __forceinline__ float f_gelu_bf(float x) {
  constexpr float kQuarterL = -3.60673760e-01f;  // -log2(e) / 4
  const float t = fabsf(x);
  const float h = __builtin_amdgcn_exp2f((t * t) * kQuarterL);
  const float e = h * h;
  const float u = __builtin_amdgcn_rcpf(__builtin_fmaf(kGeluBfP, t, 1.0f));
  float P = -1.2567331e-01f;
  P = __builtin_fmaf(P, u, 2.4604563e-01f);
  P = __builtin_fmaf(P, u, 1.7890283e-01f);
  P = __builtin_fmaf(P, u, 2.0061062e-01f);
  const float q = (e * u) * P;
  return x * (x >= 0.f ? 1.0f - q : q);
}
__device__ __forceinline__ float f_relu(float x) { return x > 0.f ? x : 0.f; }

// tanh without a lane-dependent branch (a branch inside an interpreter case
// would make the compiler linearise the whole dispatch switch): both forms
// are computed and one is selected.  |x| < 0.15: x - x^3/3 + 2x^5/15, the
// series, whose first omitted term is under 6.2e-7 of the value there;
// otherwise (1 - e) / (1 + e) with e = e^{-2|x|} = 2^(-2 log2(e) |x|) in
// one rounding of the argument.  e's relative error is multiplied by
// 2e / (1 - e^2) in the result, at most 3.3 at the branch point and
// falling beyond it, so with the hardware exp2 and reciprocal within an
// ulp each the result stays under 6.6e-7 relative everywhere (a host
// replay of every operation, each result moved by up to an ulp either way,
// over a fine grid and the subnormal range).  13 VALU slots.
__device__ __forceinline__ float f_tanh(float x) {
  const float ax = fabsf(x);
  const float u = ax * ax;
  const float p = __builtin_fmaf(u, 0.133333333f, -0.333333343f);
  const float small = __builtin_fmaf(ax * u, p, ax);
  constexpr float kM2L = -2.88539004e+00f;  // -2 log2(e)
  const float e = __builtin_amdgcn_exp2f(ax * kM2L);
  const float big = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
  return copysignf(ax < 0.15f ? small : big, x);
}

// ---------------------------------------------------------------- predicated stores
// A store for the lanes in `mask` only, without a branch: EXEC is narrowed
// for the one instruction.  Partial tiles and the reduce tail write this
// way so that the element loop holds no lane-dependent branch.
__device__ __forceinline__ void pstore_b32(void* addr, uint32_t v, uint64_t mask) {
  uint64_t save;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b64 exec, exec, %3\n\t"
      "global_store_dword %1, %2, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(save)
      : "v"(addr), "v"(v), "s"(mask));
}
__device__ __forceinline__ void pstore_b16(void* addr, uint32_t v, uint64_t mask) {
  uint64_t save;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_and_b64 exec, exec, %3\n\t"
      "global_store_short %1, %2, off\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(save)
      : "v"(addr), "v"(v), "s"(mask));
}
__device__ __forceinline__ uint64_t lanes(bool c) { return __builtin_amdgcn_ballot_w64(c); }

// A wave-uniform value the compiler must treat as produced right here: the
// tests and arithmetic on it that follow cannot be hoisted out of the
// enclosing loop.  The executor's loop-invariant conditions, hoisted, each
// hold a pair of SGPRs for the whole kernel; past the SGPR budget they are
// spilled to VGPR lanes.  Recomputing one is a scalar compare.
template <typename T>
__device__ __forceinline__ T here(T x) {
  asm volatile("" : "+s"(x));
  return x;
}
// The same for a per-lane value (lane masks derived from the lane index).
__device__ __forceinline__ int here_lane(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// ---------------------------------------------------------------- context
// A lane's tile.  In the whole-tile (FAST) instance it is V / kV sub-tiles
// of kV consecutive elements, kstride elements apart in the same row; in
// the partial-tile instance it is one sub-tile of cnt valid elements.
struct Tile {
  int64_t row;   // global row
  int64_t col;   // global column of the first element
  int64_t eoff;  // element offset of the tile in [R,C] tensors
  int cl;        // column inside the staged panel
  int rr;        // row inside the row block
  int cnt;       // valid elements of a partial tile
  int kstride;   // elements between sub-tiles
  bool valid;    // the tile exists (row and column in range)
  bool vec;      // whole sub-tile, 16-byte aligned: vector path
  SlotPtr* ptrs;      // the slots' base pointers (wave-uniform)
  uint32_t vmask;     // slots that take 16-byte accesses (wave-uniform)
};

template <int V, int MODE>
__device__ __forceinline__ int64_t elem_offset(const ExecArgs& a, int slot, const Tile& t) {
  if (MODE == M_ELEM) return t.eoff;
  if (MODE == M_ROW) return t.row * a.rstride[slot];
  return t.col * a.cstride[slot];
}

__device__ __forceinline__ void expand_bf16(float* d, u4 w) {
  d[0] = bf16_lo(w.x); d[1] = bf16_hi(w.x); d[2] = bf16_lo(w.y); d[3] = bf16_hi(w.y);
  d[4] = bf16_lo(w.z); d[5] = bf16_hi(w.z); d[6] = bf16_lo(w.w); d[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void expand_u8(float* d, u2 w) {
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = (float)((w.x >> (8 * i)) & 0xFFu);
#pragma unroll
  for (int i = 0; i < 4; ++i) d[4 + i] = (float)((w.y >> (8 * i)) & 0xFFu);
}

// Loads.  Element phase: whole tiles use one 16-byte load per sub-tile
// (u8: 8 bytes) when the slot is aligned for it, else one load per
// element; partial tiles read element by element at clamped in-range
// indices, without a branch.  Column phase (V = kV): a tile is kV
// consecutive columns of a [C] tensor (cstride 1), or one [1,1] value
// (cstride 0) broadcast.  Row phase (V = 1): one element.
// A slot whose pointer (and, for [R,C] tensors, row pitch) allows 16-byte
// accesses (u8: 8-byte); the host sets one bit per slot (per set in a
// multi-set run).
__device__ __forceinline__ bool slot_vec(const Tile& t, int slot) {
  return (t.vmask >> slot) & 1u;
}
template <int V, int MODE>
__device__ __forceinline__ bool tile_mode() {
  return MODE == M_ELEM || (MODE == M_COL && V > 1);
}
template <int V, int MODE>
__device__ __forceinline__ int64_t tile_base(const Tile& t) {
  return MODE == M_ELEM ? t.eoff : t.col;
}

__device__ __forceinline__ float bf16_g(const GAS uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }

// Streamed element tiles are read with nontemporal loads: data read once
// need not displace what the caches hold for reuse (broadcast panels, the
// op program), and on this part streaming loads reach a higher share of
// HBM bandwidth (the stream probes: reads 7.0 TB/s against 6.2 with
// ordinary loads).
__device__ __forceinline__ u4 ld_nt16(const GAS void* p) {
  return __builtin_nontemporal_load((const GAS u4*)p);
}
__device__ __forceinline__ f4 ld_nt16f(const GAS void* p) {
  return __builtin_nontemporal_load((const GAS f4*)p);
}
__device__ __forceinline__ u2 ld_nt8(const GAS void* p) {
  return __builtin_nontemporal_load((const GAS u2*)p);
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void load_f32(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const GAS float* b = (const GAS float*)t.ptrs[slot];
  if (tile_mode<V, MODE>()) {
    if (MODE == M_COL && a.cstride[slot] == 0) {
      const float x = b[0];
#pragma unroll
      for (int i = 0; i < V; ++i) d[i] = x;
      return;
    }
    const int64_t base = tile_base<V, MODE>(t);
    if ((FAST || t.vec) && slot_vec(t, slot)) {
      const GAS float* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k) {
        const f4 x = MODE == M_ELEM ? ld_nt16f(p + k * here(t.kstride)) : *(const GAS f4*)(p + k * here(t.kstride));
        const f4 y = MODE == M_ELEM ? ld_nt16f(p + k * here(t.kstride) + 4)
                                    : *(const GAS f4*)(p + k * here(t.kstride) + 4);
        d[k * kV + 0] = x.x; d[k * kV + 1] = x.y; d[k * kV + 2] = x.z; d[k * kV + 3] = x.w;
        d[k * kV + 4] = y.x; d[k * kV + 5] = y.y; d[k * kV + 6] = y.z; d[k * kV + 7] = y.w;
      }
      return;
    }
    if (FAST || t.vec) {  // whole tile, element-aligned only
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
#pragma unroll
        for (int i = 0; i < kV; ++i) d[k * kV + i] = b[base + k * here(t.kstride) + i];
      return;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = b[(t.valid && i < t.cnt) ? base + i : 0];
    return;
  }
  d[0] = b[elem_offset<V, MODE>(a, slot, t)];
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void load_bf16(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const GAS uint16_t* b = (const GAS uint16_t*)t.ptrs[slot];
  if (tile_mode<V, MODE>()) {
    if (MODE == M_COL && a.cstride[slot] == 0) {
      const float x = bf16_g(b);
#pragma unroll
      for (int i = 0; i < V; ++i) d[i] = x;
      return;
    }
    const int64_t base = tile_base<V, MODE>(t);
    if ((FAST || t.vec) && slot_vec(t, slot)) {
      const GAS uint16_t* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
        expand_bf16(d + k * kV, MODE == M_ELEM ? ld_nt16(p + k * here(t.kstride))
                                               : *(const GAS u4*)(p + k * here(t.kstride)));
      return;
    }
    if (FAST || t.vec) {  // whole tile, element-aligned only
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
#pragma unroll
        for (int i = 0; i < kV; ++i) d[k * kV + i] = bf16_g(b + base + k * here(t.kstride) + i);
      return;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = bf16_g(b + ((t.valid && i < t.cnt) ? base + i : 0));
    return;
  }
  d[0] = bf16_g(b + elem_offset<V, MODE>(a, slot, t));
}

// Addressed loads.  Element j of a tile sits at row t.row, column
// t.col + (j / kV) * kstride + j % kV; a transposed source is read there at
// row * rstride + col * cstride, one element per load.  A concat reads
// columns left of the split from slot arg & 0xFF and the rest, shifted by
// the split, from slot arg >> 8.  Elements outside a partial tile read the
// first element of the first slot.
template <bool BF>
__device__ __forceinline__ float load_one(const void* base, int64_t off) {
  if (BF) return bf16_g((const GAS uint16_t*)base + off);
  return ((const GAS float*)base)[off];
}
template <int V, int MODE, bool FAST, bool BF>
__device__ __forceinline__ void load_gather(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const void* base = t.ptrs[slot];
  const int64_t rowoff = t.row * a.rstride[slot], cs = a.cstride[slot];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j % kV;
    const bool ok = FAST || (t.valid && i < t.cnt);
    const int64_t col = t.col + (int64_t)(j / kV) * t.kstride + i;
    d[j] = load_one<BF>(base, ok ? rowoff + col * cs : 0);
  }
}
template <int V, int MODE, bool FAST, bool BF>
__device__ __forceinline__ void load_concat(float (&d)[V], const ExecArgs& a, int arg, float split_f,
                                            const Tile& t) {
  const int sa = arg & 0xFF, sb = arg >> 8;
  const int64_t split = (int64_t)split_f;
  const void* pa = t.ptrs[sa];
  const void* pb = t.ptrs[sb];
  const int64_t ra = t.row * a.rstride[sa], rb = t.row * a.rstride[sb];
  const int64_t ca = a.cstride[sa], cb = a.cstride[sb];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int i = j % kV;
    const bool ok = FAST || (t.valid && i < t.cnt);
    const int64_t col = t.col + (int64_t)(j / kV) * t.kstride + i;
    const bool left = !ok || col < split;
    const int64_t off = !ok ? 0 : left ? ra + col * ca : rb + (col - split) * cb;
    d[j] = load_one<BF>(left ? pa : pb, off);
  }
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void load_u8(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const GAS uint8_t* b = (const GAS uint8_t*)t.ptrs[slot];
  if (tile_mode<V, MODE>()) {
    if (MODE == M_COL && a.cstride[slot] == 0) {
      const float x = (float)b[0];
#pragma unroll
      for (int i = 0; i < V; ++i) d[i] = x;
      return;
    }
    const int64_t base = tile_base<V, MODE>(t);
    if ((FAST || t.vec) && slot_vec(t, slot)) {
      const GAS uint8_t* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
        expand_u8(d + k * kV, MODE == M_ELEM ? ld_nt8(p + k * here(t.kstride))
                                             : *(const GAS u2*)(p + k * here(t.kstride)));
      return;
    }
    if (FAST || t.vec) {  // whole tile, element-aligned only
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
#pragma unroll
        for (int i = 0; i < kV; ++i) d[k * kV + i] = (float)b[base + k * here(t.kstride) + i];
      return;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = (float)b[(t.valid && i < t.cnt) ? base + i : 0];
    return;
  }
  d[0] = (float)b[elem_offset<V, MODE>(a, slot, t)];
}

// Stores: whole tiles 16 bytes per sub-tile (one store per element when
// the slot is not 16-byte aligned); partial tiles one predicated store per
// element.  A column-phase store writes a [1,C] output (cstride
// 1) and runs only in the workgroups of the first row block.
template <int V, int MODE, bool FAST>
__device__ __forceinline__ void store_f32(const float (&s)[V], const ExecArgs& a, int slot, const Tile& t) {
  GAS float* b = (GAS float*)t.ptrs[slot];
  if (tile_mode<V, MODE>()) {
    const int64_t base = tile_base<V, MODE>(t);
    if ((FAST || t.vec) && slot_vec(t, slot)) {
      GAS float* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k) {
        const f4 x = {s[k * kV], s[k * kV + 1], s[k * kV + 2], s[k * kV + 3]};
        const f4 y = {s[k * kV + 4], s[k * kV + 5], s[k * kV + 6], s[k * kV + 7]};
        *(GAS f4*)(p + k * here(t.kstride)) = x;
        *(GAS f4*)(p + k * here(t.kstride) + 4) = y;
      }
      return;
    }
    if (FAST || t.vec) {  // whole tile, element-aligned only
      GAS float* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
#pragma unroll
        for (int i = 0; i < kV; ++i) p[k * here(t.kstride) + i] = s[k * kV + i];
      return;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool on = t.valid && i < t.cnt;
      pstore_b32((void*)(b + (on ? base + i : 0)), __float_as_uint(s[i]), lanes(on));
    }
    return;
  }
  b[elem_offset<V, MODE>(a, slot, t)] = s[0];
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void store_bf16(const float (&s)[V], const ExecArgs& a, int slot, const Tile& t) {
  GAS uint16_t* b = (GAS uint16_t*)t.ptrs[slot];
  if (tile_mode<V, MODE>()) {
    const int64_t base = tile_base<V, MODE>(t);
    if ((FAST || t.vec) && slot_vec(t, slot)) {
      GAS uint16_t* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k) {
        const u4 w = {pack2_bf16(s[k * kV], s[k * kV + 1]), pack2_bf16(s[k * kV + 2], s[k * kV + 3]),
                      pack2_bf16(s[k * kV + 4], s[k * kV + 5]), pack2_bf16(s[k * kV + 6], s[k * kV + 7])};
        *(GAS u4*)(p + k * here(t.kstride)) = w;
      }
      return;
    }
    if (FAST || t.vec) {  // whole tile, element-aligned only
      GAS uint16_t* p = b + base;
#pragma unroll
      for (int k = 0; k < V / kV; ++k)
#pragma unroll
        for (int i = 0; i < kV; ++i) p[k * here(t.kstride) + i] = (uint16_t)(pack_bf16(s[k * kV + i], 0.f) & 0xFFFFu);
      return;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool on = t.valid && i < t.cnt;
      pstore_b16((void*)(b + (on ? base + i : 0)), pack_bf16(s[i], 0.f) & 0xFFFFu, lanes(on));
    }
    return;
  }
  b[elem_offset<V, MODE>(a, slot, t)] = (uint16_t)(pack_bf16(s[0], 0.f) & 0xFFFFu);
}

// ---------------------------------------------------------------- row accumulators
// A lane's share of the row reduction its stage ends in.  a is the sum
// (row_sum, row_mean) or the largest value (row_max).  The paired
// reductions carry two results in one pass over the row:
//  * mean and variance: a = mean, b = sum of squared deviations from it,
//    c = count, merged by the pairwise update of Chan, Golub and LeVeque
//    (1979) (a parallel form of Welford's);
//  * max and sum of exponentials: a = largest value, b = sum of
//    exp(x - a), the sum rescaled by exp(a_old - a_new) as the maximum grows.
struct RowAcc {
  float a, b, c;
};

// x then y (the order fixes the rounding; callers keep it canonical).  An
// empty side (count 0, or max -inf) leaves the other as it is.
__device__ __forceinline__ RowAcc merge_mv(RowAcc x, RowAcc y) {
  const float n = x.c + y.c;
  const float w = y.c / n;
  const float d = y.a - x.a;
  RowAcc r;
  r.a = x.a + d * w;
  r.b = (x.b + y.b) + (d * d) * (x.c * w);
  r.c = n;
  return n > 0.f ? r : x;
}
__device__ __forceinline__ RowAcc merge_se(RowAcc x, RowAcc y) {
  const float m = fmaxf(x.a, y.a);
  // an empty side's -inf would give exp_nonpos(-inf - m): select 0 instead
  const float fx = x.a == -INFINITY ? 0.f : exp_nonpos(x.a - m);
  const float fy = y.a == -INFINITY ? 0.f : exp_nonpos(y.a - m);
  RowAcc r;
  r.a = m;
  r.b = x.b * fx + y.b * fy;
  r.c = 0.f;
  return m == -INFINITY ? x : r;
}

// ---------------------------------------------------------------- ops
// d = f(s) element by element (d and s may be the same register)
template <int V, int F>
__device__ __forceinline__ void unary(float (&d)[V], const float (&s)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float x = s[i];
    float y;
    if (F == F_EXP) y = f_exp(x);
    else if (F == F_TANH) y = f_tanh(x);
    else if (F == F_SIGMOID) y = f_sigmoid(x);
    else if (F == F_RELU) y = f_relu(x);
    else if (F == F_GELU) y = f_gelu(x);
    else if (F == F_GELU_BF) y = f_gelu_bf(x);
    else if (F == F_SQUARE) y = x * x;
    else if (F == F_SQRT) y = sqrtf(x);
    else if (F == F_RECIP) y = 1.0f / x;
    else y = -x;  // F_NEG
    d[i] = y;
  }
}

template <int OP>
__device__ __forceinline__ float xop(float v, float x) {
  if (OP == X_ADD) return v + x;
  if (OP == X_SUB) return v - x;
  if (OP == X_RSUB) return x - v;
  if (OP == X_MUL) return v * x;
  if (OP == X_DIV) return v / x;
  if (OP == X_RDIV) return x / v;
  if (OP == X_MAX) return fmaxf(v, x);
  return fminf(v, x);  // X_MIN
}

template <int V, int OP>
__device__ __forceinline__ void binop(float (&l)[V], const float (&r)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) l[i] = xop<OP>(l[i], r[i]);
}

// A tile's column-broadcast values from an LDS column slot: kV consecutive
// fp32 values per sub-tile (32-byte aligned), sub-tiles kstride apart.
template <int V>
__device__ __forceinline__ void lds_vec(float (&d)[V], const float* x, int kstride) {
  if (V % kV == 0) {
#pragma unroll
    for (int k = 0; k < V / kV; ++k) {
      const float4 u = *(const float4*)(x + k * kstride);
      const float4 w = *(const float4*)(x + k * kstride + 4);
      d[k * kV + 0] = u.x; d[k * kV + 1] = u.y; d[k * kV + 2] = u.z; d[k * kV + 3] = u.w;
      d[k * kV + 4] = w.x; d[k * kV + 5] = w.y; d[k * kV + 6] = w.z; d[k * kV + 7] = w.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = x[i];
  }
}

// V values of one row of the staged transposed tile (row stride PW + 1,
// so only 4-byte aligned): sub-tile k at x + k * kstride.
template <int V>
__device__ __forceinline__ void lds_tile(float (&d)[V], const float* x, int kstride) {
#pragma unroll
  for (int j = 0; j < V; ++j) d[j] = x[(j / kV) * kstride + j % kV];
}

// A op (column values), one sub-tile at a time: a scheduling barrier
// between sub-tiles keeps the compiler from reading all V values from LDS
// ahead of the arithmetic, which would hold V more registers.
template <int V, int OP>
__device__ __forceinline__ void xvec(float (&r)[V], const float* x, int kstride) {
  if (V % kV == 0) {
#pragma unroll
    for (int k = 0; k < V / kV; ++k) {
      float xs[kV];
      lds_vec<kV>(xs, x + k * kstride, 0);
#pragma unroll
      for (int i = 0; i < kV; ++i) r[k * kV + i] = xop<OP>(r[k * kV + i], xs[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] = xop<OP>(r[i], x[i]);
  }
}

template <int V, int OP>
__device__ __forceinline__ void xscalar(float (&r)[V], float x) {
#pragma unroll
  for (int i = 0; i < V; ++i) r[i] = xop<OP>(r[i], x);
}
template <int V, int OP>
__device__ __forceinline__ void xscalar_from(float (&d)[V], const float (&s)[V], float x) {
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = xop<OP>(s[i], x);
}

template <int V>
__device__ __forceinline__ void copy(float (&d)[V], const float (&s)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = s[i];
}

template <int V>
__device__ __forceinline__ void fill(float (&d)[V], float x) {
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = x;
}

// ---------------------------------------------------------------- interpreter
// A, B and the NS spill slots hold one tile each (V values per lane).  The
// next instruction word is fetched while the current one executes.  FAST is
// the instance for tiles that are whole, in range and vector-aligned in
// every lane of the wave: it has no lane-dependent branch, so the compiler
// keeps the dispatch switch a tree of scalar branches (a lane-dependent
// branch anywhere in the loop makes it linearise the switch into a chain of
// guarded blocks).  The other instance handles partial sub-tiles at row and
// tensor ends.  Forms naming a slot beyond NS never occur in a program
// compiled for the instance and have empty bodies.
// run_prog executes instructions [pc0, n) on registers the caller owns, so
// a program can be started before a phase barrier (its leading loads) and
// finished after it; interpret runs a whole program on its own registers.
template <int V, int MODE, bool FAST, int NS, bool TR = false>
__device__ __forceinline__ void run_prog(const ExecArgs& a, const Instr* prog, int pc0, int n,
                                         const Tile& t, float (&A)[V], float (&B)[V],
                                         float (&S)[NS > 0 ? NS : 1][V], float* lds_col,
                                         float* lds_row, RowAcc& acc, bool store_global) {
  if (pc0 >= n) return;
  Instr cur = prog[pc0];
  for (int pc = pc0; pc < n; ++pc) {
    const Instr nxt = prog[pc + 1 < n ? pc + 1 : pc];
    const int arg = cur.arg;
    const float* col = lds_col + arg * a.PW + t.cl;
    switch (cur.code) {
      case F_LD_F32_A: load_f32<V, MODE, FAST>(A, a, arg, t); break;
      case F_LD_BF16_A: load_bf16<V, MODE, FAST>(A, a, arg, t); break;
      case F_LD_U8_A: load_u8<V, MODE, FAST>(A, a, arg, t); break;
      case F_LD_F32_B: load_f32<V, MODE, FAST>(B, a, arg, t); break;
      case F_LD_BF16_B: load_bf16<V, MODE, FAST>(B, a, arg, t); break;
      case F_LD_U8_B: load_u8<V, MODE, FAST>(B, a, arg, t); break;
      // addressed loads exist only for one sub-tile at a time (a program
      // holding one runs with slow_only set, never on the whole-run path)
      case F_LDG_F32_A:
        if constexpr (MODE == M_ELEM && V == kV) load_gather<V, MODE, FAST, false>(A, a, arg, t);
        break;
      case F_LDG_BF16_A:
        if constexpr (MODE == M_ELEM && V == kV) load_gather<V, MODE, FAST, true>(A, a, arg, t);
        break;
      case F_LDC_F32_A:
        if constexpr (MODE != M_ROW && V == kV) load_concat<V, MODE, FAST, false>(A, a, arg, cur.imm, t);
        break;
      case F_LDC_BF16_A:
        if constexpr (MODE != M_ROW && V == kV) load_concat<V, MODE, FAST, true>(A, a, arg, cur.imm, t);
        break;
      case F_LDT_A:
        if constexpr (MODE == M_ELEM && TR) lds_tile<V>(A, lds_col + a.tr_off + t.rr * a.tr_stride + t.cl, t.kstride);
        break;
      case F_COL_A: if (MODE == M_ELEM) lds_vec<V>(A, col, t.kstride); break;
      case F_ROW_A: if (MODE != M_COL) fill<V>(A, lds_row[arg * a.RB + t.rr]); break;
      case F_IMM_A: fill<V>(A, cur.imm); break;
      case F_COL_B: if (MODE == M_ELEM) lds_vec<V>(B, col, t.kstride); break;
      case F_ROW_B: if (MODE != M_COL) fill<V>(B, lds_row[arg * a.RB + t.rr]); break;
      case F_IMM_B: fill<V>(B, cur.imm); break;
      case F_A2B: copy<V>(B, A); break;
      case F_B2A: copy<V>(A, B); break;
#define GTF_SLOT(K)                                                 \
  case F_A2S0 + K: if constexpr (K < NS) copy<V>(S[K], A); break;   \
  case F_B2S0 + K: if constexpr (K < NS) copy<V>(S[K], B); break;   \
  case F_S02A + K: if constexpr (K < NS) copy<V>(A, S[K]); break;   \
  case F_S02B + K: if constexpr (K < NS) copy<V>(B, S[K]); break;
      GTF_SLOT(0) GTF_SLOT(1) GTF_SLOT(2) GTF_SLOT(3) GTF_SLOT(4) GTF_SLOT(5)
#undef GTF_SLOT
#define GTF_UN(NAME) case F_##NAME: unary<V, F_##NAME>(A, A); break;
#define GTF_UN_B(NAME)                                        \
  case F_##NAME: unary<V, F_##NAME>(A, A); break;             \
  case F_##NAME##_B: unary<V, F_##NAME>(A, B); break;
      GTF_UN_B(EXP) GTF_UN_B(TANH) GTF_UN(SIGMOID) GTF_UN_B(RELU) GTF_UN(GELU) GTF_UN(GELU_BF)
      GTF_UN_B(SQUARE) GTF_UN(SQRT) GTF_UN(RECIP) GTF_UN_B(NEG)
#undef GTF_UN
#undef GTF_UN_B
#define GTF_BIN(NAME, OP)                                                               \
  case F_##NAME: binop<V, OP>(A, B); break;                                             \
  case F_##NAME##_C: if (MODE == M_ELEM) xvec<V, OP>(A, col, t.kstride); break;         \
  case F_##NAME##_R: if (MODE != M_COL) xscalar<V, OP>(A, lds_row[arg * a.RB + t.rr]); break; \
  case F_##NAME##_I: xscalar<V, OP>(A, cur.imm); break;                                \
  case F_##NAME##_IB: xscalar_from<V, OP>(A, B, cur.imm); break;
      GTF_BIN(ADD, X_ADD)
      GTF_BIN(SUB, X_SUB)
      GTF_BIN(RSUB, X_RSUB)
      GTF_BIN(MUL, X_MUL)
      GTF_BIN(DIV, X_DIV)
      GTF_BIN(RDIV, X_RDIV)
      GTF_BIN(MAX, X_MAX)
      GTF_BIN(MIN, X_MIN)
#undef GTF_BIN
      case F_ST_F32:
        if (MODE == M_ELEM || store_global) store_f32<V, MODE, FAST>(A, a, arg, t);
        break;
      case F_ST_BF16:
        if (MODE == M_ELEM || store_global) store_bf16<V, MODE, FAST>(A, a, arg, t);
        break;
      case F_RED:
        if (MODE == M_ELEM) {
#pragma unroll
          for (int i = 0; i < V; ++i) acc.a += (FAST || (t.valid && i < t.cnt)) ? A[i] : 0.f;
        }
        break;
      case F_RED_MAX:
        if (MODE == M_ELEM) {
#pragma unroll
          for (int i = 0; i < V; ++i) acc.a = fmaxf(acc.a, (FAST || (t.valid && i < t.cnt)) ? A[i] : -INFINITY);
        }
        break;
      // (the staged-transpose instance runs no reductions)
      case F_RED_MV:
        // this tile's (mean, squared deviations, count), then merged in
        if constexpr (MODE == M_ELEM && !TR) {
          float s = 0.f, cnt = 0.f;
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const bool ok = FAST || (t.valid && i < t.cnt);
            s += ok ? A[i] : 0.f;
            cnt += ok ? 1.f : 0.f;
          }
          const float m = FAST ? s * (1.0f / V) : (cnt > 0.f ? s / cnt : 0.f);
          float q = 0.f;
#pragma unroll
          for (int i = 0; i < V; ++i) {
            const float d = A[i] - m;
            q = (FAST || (t.valid && i < t.cnt)) ? __builtin_fmaf(d, d, q) : q;
          }
          acc = merge_mv(acc, RowAcc{m, q, cnt});
        }
        break;
      case F_RED_SE:
        // this tile's (max, sum of exp(x - max)), then merged in
        if constexpr (MODE == M_ELEM && !TR) {
          float m = -INFINITY;
#pragma unroll
          for (int i = 0; i < V; ++i) m = fmaxf(m, (FAST || (t.valid && i < t.cnt)) ? A[i] : -INFINITY);
          // an element at -inf adds exp(-inf) = 0; a tile of only -inf has
          // m = -inf too, where A[i] - m would be a NaN: it is taken
          // against 0 instead (one select per tile) and adds 0
          const float ms = m == -INFINITY ? 0.f : m;
          float s = 0.f;
#pragma unroll
          for (int i = 0; i < V; ++i)
            s += (FAST || (t.valid && i < t.cnt)) ? exp_nonpos(A[i] - ms) : 0.f;
          acc = merge_se(acc, RowAcc{m, s, 0.f});
        }
        break;
      case F_ST_LDS:
        if (MODE == M_ROW) lds_row[arg * a.RB + t.rr] = A[0];
        if (MODE == M_COL) {
#pragma unroll
          for (int i = 0; i < V; ++i)
            if (i < t.cnt) lds_col[arg * a.PW + t.cl + i] = A[i];
        }
        break;
      default:
        break;
    }
    cur = nxt;
  }
}

template <int V, int MODE, bool FAST, int NS, bool TR = false>
__device__ __forceinline__ void interpret(const ExecArgs& a, const Instr* prog, int n,
                                          const Tile& t, float* lds_col, float* lds_row,
                                          RowAcc& acc, bool store_global) {
  float A[V], B[V], S[NS > 0 ? NS : 1][V];
  // a program writes a register before reading it; left undefined, the
  // registers would be zeroed on every call (one move each per tile)
#pragma unroll
  for (int i = 0; i < V; ++i) asm volatile("" : "=v"(A[i]), "=v"(B[i]));
  run_prog<V, MODE, FAST, NS, TR>(a, prog, 0, n, t, A, B, S, lds_col, lds_row, acc, store_global);
}

// ---------------------------------------------------------------- reduce tail
// The value of lane ctrl_id's partner in the reduction tree (DPP).
__device__ __forceinline__ float dpp_partner(float v, int ctrl_id) {
  int x = __float_as_int(v);
  int y;
  switch (ctrl_id) {
    case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return __int_as_float(y);
}

// The sum (MAX false) or the largest value (MAX true) over aligned segments
// of `width` lanes (a power of two <= 64); every lane of a segment ends
// with the segment's result.
template <bool MAX>
__device__ __forceinline__ float red2(float a, float b) {
  return MAX ? fmaxf(a, b) : a + b;
}
template <bool MAX>
__device__ __forceinline__ float segment_reduce(float v, int width) {
  if (width >= 2) v = red2<MAX>(v, dpp_partner(v, 0));
  if (width >= 4) v = red2<MAX>(v, dpp_partner(v, 1));
  if (width >= 8) v = red2<MAX>(v, dpp_partner(v, 2));
  if (width >= 16) v = red2<MAX>(v, dpp_partner(v, 3));
  if (width >= 32) v = red2<MAX>(v, __shfl_xor(v, 16));
  if (width >= 64) v = red2<MAX>(v, __shfl_xor(v, 32));
  return v;
}

// The reduction tree for a paired accumulator (KIND 4: mean and variance,
// 5: max and sum of exponentials).  At each step a lane merges its value
// with its partner's in a fixed order, the lower-half lane's first, so
// both lanes of a pair compute the same bits and every lane of a segment
// ends with the segment's result, as in segment_reduce.
template <int KIND>
__device__ __forceinline__ RowAcc merge_kind(RowAcc x, RowAcc y) {
  return KIND == 4 ? merge_mv(x, y) : merge_se(x, y);
}
template <int KIND>
__device__ __forceinline__ RowAcc pair_step(RowAcc v, RowAcc p, bool lower) {
  return lower ? merge_kind<KIND>(v, p) : merge_kind<KIND>(p, v);
}
template <int KIND>
__device__ __forceinline__ RowAcc segment_pair(RowAcc v, int width) {
  const int lane = here_lane(threadIdx.x & 63);
  auto dpp = [&](int ctrl) {
    return RowAcc{dpp_partner(v.a, ctrl), dpp_partner(v.b, ctrl), dpp_partner(v.c, ctrl)};
  };
  auto shf = [&](int m) { return RowAcc{__shfl_xor(v.a, m), __shfl_xor(v.b, m), __shfl_xor(v.c, m)}; };
  if (width >= 2) v = pair_step<KIND>(v, dpp(0), (lane & 1) == 0);
  if (width >= 4) v = pair_step<KIND>(v, dpp(1), (lane & 2) == 0);
  if (width >= 8) v = pair_step<KIND>(v, dpp(2), (lane & 7) < 4);
  if (width >= 16) v = pair_step<KIND>(v, dpp(3), (lane & 15) < 8);
  if (width >= 32) v = pair_step<KIND>(v, shf(16), (lane & 16) == 0);
  if (width >= 64) v = pair_step<KIND>(v, shf(32), (lane & 32) == 0);
  return v;
}

// A row result, for the lanes in `on` (one lane per row): to an LDS row
// slot, where later stages and row programs read it, and/or with a
// predicated store to an external slot.
__device__ __forceinline__ void store_row(const ExecArgs& a, float* lds_row, int lds_slot, int ext_slot,
                                          int dtype, int64_t row, int rr, float v, bool on) {
  if (lds_slot >= 0 && on) lds_row[lds_slot * a.RB + rr] = v;
  if (ext_slot < 0) return;
  const int64_t off = on ? row * a.rstride[ext_slot] : 0;
  const uint64_t m = lanes(on);
  if (dtype == DT_BF16)
    pstore_b16((uint16_t*)a.ptr[ext_slot] + off, pack_bf16(v, 0.f) & 0xFFFFu, m);
  else
    pstore_b32((float*)a.ptr[ext_slot] + off, __float_as_uint(v), m);
}

// The row result(s) of a stage's reduction from the merged accumulator.
__device__ __forceinline__ void store_reduced(const ExecArgs& a, const StageDesc& S, float* lds_row,
                                              int64_t row, int rr, RowAcc r, bool on) {
  float first = r.a, second = r.b;
  if (S.red == 2) first = r.a / (float)a.C;
  if (S.red == 4) {
    first = r.c > 0.f ? r.a : __builtin_nanf("");  // an empty row's mean is 0 / 0
    second = r.b / r.c;
  }
  store_row(a, lds_row, S.red_lds, S.red_slot, S.red_dtype, row, rr, first, on);
  if (S.red >= 4) store_row(a, lds_row, S.red2_lds, S.red2_slot, S.red2_dtype, row, rr, second, on);
}

// The first 1 KiB of the kernel arguments -- the header, the stage table,
// the slot pointers and strides, and the start of the op programs -- pulled
// into the scalar cache with one scalar load per 64-byte line, all in
// flight at once, before anything reads them.  Every wave of a launch
// starts at the same moment and then walks a chain of dependent argument
// reads (item bounds, stage, instruction, slot pointer); without this each
// new line on that chain is a miss the whole chain waits for.
__device__ __forceinline__ void warm_args(const void CAS* p) {
  uint32_t d0, d1, d2, d3, d4, d5, d6, d7, d8, d9, d10, d11, d12, d13, d14, d15;
  asm volatile(
      "s_load_dword %0, %16, 0x0\n\t"
      "s_load_dword %1, %16, 0x40\n\t"
      "s_load_dword %2, %16, 0x80\n\t"
      "s_load_dword %3, %16, 0xc0\n\t"
      "s_load_dword %4, %16, 0x100\n\t"
      "s_load_dword %5, %16, 0x140\n\t"
      "s_load_dword %6, %16, 0x180\n\t"
      "s_load_dword %7, %16, 0x1c0\n\t"
      "s_load_dword %8, %16, 0x200\n\t"
      "s_load_dword %9, %16, 0x240\n\t"
      "s_load_dword %10, %16, 0x280\n\t"
      "s_load_dword %11, %16, 0x2c0\n\t"
      "s_load_dword %12, %16, 0x300\n\t"
      "s_load_dword %13, %16, 0x340\n\t"
      "s_load_dword %14, %16, 0x380\n\t"
      "s_load_dword %15, %16, 0x3c0\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&s"(d0), "=&s"(d1), "=&s"(d2), "=&s"(d3), "=&s"(d4), "=&s"(d5), "=&s"(d6), "=&s"(d7),
        "=&s"(d8), "=&s"(d9), "=&s"(d10), "=&s"(d11), "=&s"(d12), "=&s"(d13), "=&s"(d14), "=&s"(d15)
      : "s"(p));
}

// ---------------------------------------------------------------- executor
// K sub-tiles per lane tile, NS spill slots (see isa.h).  Lane tiles of an
// item are visited as q = (pass, s): pass = which rows of the block, s =
// which run of K sub-tiles along the row; sub-tile k of run s sits at
// column (lane_in_row + (s * K + k) * tpr) * kV.  A run whose K sub-tiles
// are whole in every lane of the wave goes to the FAST instance at once;
// any other run goes sub-tile by sub-tile to the partial instance.  Either
// way each lane adds its elements to the row accumulator in the same order.
// A group with row-resident reductions walks the item once per stage,
// with a row program (and barriers) between stages.
template <int K, int NS, bool TR>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(NS == 0 ? 4 : 3)))
exec_kernel(const ExecArgs a_in) {
  // The arguments are read through a pointer the compiler takes as new at
  // every item (here()): the header fields and what is derived from them are
  // then loaded from the scalar cache where they are used, not held in
  // SGPRs across the whole kernel (and spilled).
  typedef const ExecArgs CAS KArgs;
  KArgs* const ka = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();  // a_in is the first argument
  static_assert(sizeof(ExecArgs) >= 0x400, "the warmed lines lie inside the arguments");
  warm_args(ka);
  extern __shared__ float lds[];
  bool staged = false;
  RowAcc dummy{0.f, 0.f, 0.f};

  for (int64_t item = blockIdx.x; item < a_in.n_items; item += gridDim.x) {
    const ExecArgs& a = *(const ExecArgs*)(KArgs*)here((uint64_t)ka);
    float* lds_col = lds;
    float* lds_row = lds + a.n_col_slots * a.PW;
    float* lds_red = lds_row + a.n_row_slots * a.RB;
    const int tid = threadIdx.x;
    const int tpr = 1 << a.tpr_log2;
    const int rpp = kBlock >> a.tpr_log2;
    const int sub = tid >> a.tpr_log2;
    const int lt = tid & (tpr - 1);
    const Instr* col_prog = a.prog;
    const int64_t erow_stride = a.R == 1 ? 0 : a.C;
    const int ks = tpr * kV;  // elements between a lane's sub-tiles
    int64_t rb, r0, c0;
    int p, nr, nc;
    SlotPtr* ptrs = (SlotPtr*)a.ptr;
    uint32_t vmask = a.vec_slots;
    if (a.m_items != nullptr) {
      // multi-set run of a flat group: this item's elements of its set
      const MultiItem mi = a.m_items[item];
      rb = 0;
      p = 0;
      r0 = 0;
      nr = 1;
      c0 = mi.off;
      nc = mi.n;
      ptrs = (SlotPtr*)(a.m_ptrs + (int64_t)mi.set * a.n_slots);
      vmask = a.m_vec[mi.set];
    } else {
      // (one panel: no division)
      rb = a.n_panels == 1 ? item : item / a.n_panels;
      p = (int)(item - rb * a.n_panels);
      r0 = rb * a.RB;
      nr = (int)min((int64_t)a.RB, a.R - r0);
      c0 = (int64_t)p * a.PW;
      nc = (int)min((int64_t)a.PW, a.C - c0);
    }

    const bool col_now = a.n_col > 0 && (a.n_panels > 1 || !staged);
    // rpp and ks are powers of two: shifts, not divisions
    static_assert(kBlock == 256 && kV == 8, "the shifts below take log2(kBlock) = 8, log2(kV) = 3");
    const int npass = (nr + rpp - 1) >> (8 - a.tpr_log2);
    const int tpl = max(1, (nc + ks - 1) >> (a.tpr_log2 + 3));  // sub-tiles per lane per row
    const int spl = (tpl + K - 1) / K;                          // runs of K per lane per row
    const int nq = npass * spl;
    // later stages write LDS row slots that the previous item's last stage
    // may still be reading
    if (a.n_stages > 1) __syncthreads();

    // one walk of the item per stage
    auto run_stage = [&](const int st) __attribute__((always_inline)) {
      const StageDesc& S = a.stage[st];
      const bool row_now = S.row_len > 0;
      // Column phase (kV consecutive columns per thread per pass, from
      // thread 0 up, once) and the stage's row program (one row per thread,
      // from the last thread down) share one barrier pair, so their loads
      // overlap too.  A later stage always starts behind a barrier: its
      // row program and element program read the previous stage's results.
      if ((st == 0 && (col_now || TR)) || row_now || st > 0) {
        __syncthreads();
        if constexpr (TR) {
          // the item's tile of the transposed source X: tile row rr holds
          // X[c0 + cl][r0 + rr] at column cl (row stride PW + 1, so a
          // wave's column writes fall in different banks).  Thread tid
          // covers row rr = tid % RB and columns tid / RB, + kBlock / RB,
          // ...: consecutive threads read consecutive elements of one X
          // row, a wave whole 64-element runs.
          if (st == 0 && a.tr_bf16 && a.tr_vec && nr == a.RB) {
            // whole row blocks of a 16-byte aligned bf16 source: each
            // thread reads 8 consecutive elements (rows rr8 .. rr8 + 7 of
            // the tile) of one X row with one 16-byte load
            const int per = a.RB >> 3;                  // threads per X row
            const int rr8 = (tid & (per - 1)) << 3;
            const int step = kBlock / per;
            const int64_t xrow = a.cstride[a.tr_slot];
            const GAS uint16_t* src = (const GAS uint16_t*)ptrs[a.tr_slot] + c0 * xrow + r0 + rr8;
            float* dst = lds + a.tr_off + rr8 * a.tr_stride;
            for (int cl = tid / per; cl < a.PW; cl += step) {
              float v[kV];
              if (cl < nc) {
                expand_bf16(v, *(const GAS u4*)(src + cl * xrow));
              } else {
#pragma unroll
                for (int i = 0; i < kV; ++i) v[i] = 0.f;
              }
#pragma unroll
              for (int i = 0; i < kV; ++i) dst[i * a.tr_stride + cl] = v[i];
            }
          } else if (st == 0) {
            const int rr = tid & (a.RB - 1);
            const int step = kBlock >> (8 - a.tpr_log2);  // kBlock / RB
            const int64_t xrow = a.cstride[a.tr_slot];
            float* dst = lds + a.tr_off + rr * a.tr_stride;
            const bool row_ok = rr < nr;
            if (a.tr_bf16) {
              const GAS uint16_t* src = (const GAS uint16_t*)ptrs[a.tr_slot] + c0 * xrow + r0 + rr;
              for (int cl = tid >> (8 - a.tpr_log2); cl < a.PW; cl += step)
                dst[cl] = row_ok && cl < nc ? bf16_g(src + cl * xrow) : 0.f;
            } else {
              const GAS float* src = (const GAS float*)ptrs[a.tr_slot] + c0 * xrow + r0 + rr;
              for (int cl = tid >> (8 - a.tpr_log2); cl < a.PW; cl += step)
                dst[cl] = row_ok && cl < nc ? src[cl * xrow] : 0.f;
            }
          }
        }
        if (st == 0 && col_now) {
          for (int c = here_lane(tid) * kV; c < nc; c += kBlock * kV) {
            const int cnt = min(kV, nc - c);
            Tile t{0, c0 + c, 0, c, 0, cnt, 0, true, cnt == kV, ptrs, vmask};
            interpret<kV, M_COL, false, NS>(a, col_prog, a.n_col, t, lds_col, lds_row, dummy, rb == 0);
          }
          staged = true;
        }
        if (row_now) {
          for (int r = kBlock - 1 - here_lane(tid); r < nr; r += kBlock) {
            Tile t{r0 + r, 0, 0, 0, r, 1, 0, false, false, ptrs, vmask};
            interpret<1, M_ROW, false, NS>(a, a.prog + S.row_off, S.row_len, t, lds_col, lds_row,
                                           dummy, p == 0);
          }
        }
        __syncthreads();
      }
      const Instr* el_prog = a.prog + S.el_off;
      const int n_el = S.el_len;
      if (n_el == 0) return;

      // the row accumulator starts at the reduction's identity
      const bool rmax = S.red == 3 || S.red == 5;
      const RowAcc ident{rmax ? -INFINITY : 0.f, 0.f, 0.f};
      RowAcc acc = ident;
      int pass = 0, s = 0;
      // reduce tail after the last run of a row, then advance (pass, s)
      auto finish = [&](int rr) {
        if (S.red && s == spl - 1) {
          // the tail's derived values are made here, at each use, rather
          // than hoisted to the item and held in SGPRs (spilled) over it
          const int tp = here(tpr);
          const int w = min(tp, 64);
          RowAcc r = acc;
          const bool paired = !TR && S.red >= 4;  // the staged-transpose instance runs no reductions
          if (paired && S.red == 4) r = segment_pair<4>(acc, w);
          else if (paired) r = segment_pair<5>(acc, w);
          else r.a = S.red == 3 ? segment_reduce<true>(acc.a, w) : segment_reduce<false>(acc.a, w);
          acc = ident;
          if (tp > 64) {
            // rows wider than a wave: combine the per-wave results through
            // LDS in a fixed order (every lane of a wave holds the same
            // result and writes it; every lane reads those of its own row)
            const int wpr = tp >> 6;  // waves per row
            float* cell = lds_red + (here_lane(tid) >> 6) * 3;
            cell[0] = r.a;
            cell[1] = r.b;
            cell[2] = r.c;
            __syncthreads();
            const float* rowc = lds_red + sub * wpr * 3;
            RowAcc tot = ident;
            for (int k = 0; k < wpr; ++k) {
              const RowAcc x{rowc[3 * k], rowc[3 * k + 1], rowc[3 * k + 2]};
              if (paired && S.red == 4) tot = merge_mv(tot, x);
              else if (paired) tot = merge_se(tot, x);
              else tot.a = rmax ? fmaxf(tot.a, x.a) : tot.a + x.a;
            }
            r = tot;
          }
          store_reduced(a, S, lds_row, r0 + rr, rr, r, here_lane(lt) == 0 && rr < here(nr));
          if (tp > 64) __syncthreads();
        }
        if (++s == spl) {
          s = 0;
          ++pass;
        }
      };
      for (int q = 0; q < nq; ++q) {
        const int rr = pass * rpp + sub;
        const int cl0 = (lt + s * K * tpr) * kV;
        const bool row_ok = rr < nr;
        const bool whole = row_ok && cl0 + (K - 1) * ks + kV <= nc;
        // both branches are wave-uniform
        if (!a.slow_only && __all(whole)) {
          Tile t;
          t.valid = true;
          t.vec = true;
          t.row = r0 + rr;
          t.col = c0 + cl0;
          t.eoff = t.row * erow_stride + t.col;
          t.cl = cl0;
          t.rr = rr;
          t.cnt = kV;
          t.kstride = ks;
          t.ptrs = ptrs;
          t.vmask = vmask;
          interpret<K * kV, M_ELEM, true, NS, TR>(a, el_prog, n_el, t, lds_col, lds_row, acc, true);
        } else {
#pragma unroll 1
          for (int k = 0; k < K; ++k) {
            const int cl = cl0 + k * ks;
            const bool valid = row_ok && cl < nc;
            if (!__any(valid)) continue;
            Tile t;
            t.valid = valid;
            t.row = r0 + rr;
            t.col = c0 + cl;
            t.eoff = t.row * erow_stride + t.col;
            t.cl = cl;
            t.rr = rr;
            t.cnt = min(kV, nc - cl);
            t.vec = valid && t.cnt == kV;
            t.kstride = ks;
            t.ptrs = ptrs;
            t.vmask = vmask;
            interpret<kV, M_ELEM, false, NS, TR>(a, el_prog, n_el, t, lds_col, lds_row, acc, true);
          }
        }
        finish(rr);
      }
    };
    for (int st = 0; st < a.n_stages; ++st) run_stage(st);
  }
}

template __global__ void exec_kernel<kWideK, 0, false>(const ExecArgs a);
template __global__ void exec_kernel<kWideK, 0, true>(const ExecArgs a);
template __global__ void exec_kernel<kWideK, kWideNS, false>(const ExecArgs a);
template __global__ void exec_kernel<1, kNS, false>(const ExecArgs a);

// ---------------------------------------------------------------- buckets
// One workgroup per chunk: a run of up to kChunkBytes bytes of one tensor
// copied to or from its place in its bucket, times the scale.  The side that
// lives in the bucket is usually not 16-byte aligned (offsets are dense), so
// a few head elements bring the destination to a 16-byte boundary, the body
// moves 16 bytes per lane per step, and a tail finishes.  A whole chunk's
// body is one round of kU loads per thread, all in flight before the first
// store, and the workgroup then exits: on this part one short-lived
// workgroup per 16 KiB moved faster than workgroups that loop (the packing
// of 194 gradients, 151M fp32 elements, 5.7 -> 6.2 TB/s against 64 KiB
// chunks in rounds of four).  The body's loads and stores are nontemporal:
// every byte is read once and written once (nontemporal stores took the
// same packing from 5.3 to 5.7 TB/s).
template <typename T>
__device__ __forceinline__ T scale_elem(T v, float s, bool one);

template <>
__device__ __forceinline__ float scale_elem<float>(float v, float s, bool one) {
  return one ? v : v * s;
}
template <>
__device__ __forceinline__ uint16_t scale_elem<uint16_t>(uint16_t v, float s, bool one) {
  if (one) return v;
  return (uint16_t)(pack_bf16(__uint_as_float((uint32_t)v << 16) * s, 0.f) & 0xFFFFu);
}

template <typename T>
__device__ __forceinline__ uint4 scale_vec(uint4 w, float s, bool one) {
  if (one) return w;
  if (sizeof(T) == 4) {
    return make_uint4(__float_as_uint(__uint_as_float(w.x) * s), __float_as_uint(__uint_as_float(w.y) * s),
                      __float_as_uint(__uint_as_float(w.z) * s), __float_as_uint(__uint_as_float(w.w) * s));
  }
  return make_uint4(pack_bf16(bf16_lo(w.x) * s, bf16_hi(w.x) * s),
                    pack_bf16(bf16_lo(w.y) * s, bf16_hi(w.y) * s),
                    pack_bf16(bf16_lo(w.z) * s, bf16_hi(w.z) * s),
                    pack_bf16(bf16_lo(w.w) * s, bf16_hi(w.w) * s));
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16 bytes from the run's source side, which is aligned only to its element
// (4 bytes for fp32, 2 for bf16; the destination side is the one the head
// aligns to 16 bytes).  The 4-byte alignment the type declares keeps the
// load one dwordx4; the part's memory system serves such loads at 2-byte
// alignment too (the bf16 bucket tests put sources at both alignments).
// Nontemporal: every byte is read once (see ld_nt16).
typedef unsigned int u4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ uint4 load16(const void* p) {
  const u4_a4 v = __builtin_nontemporal_load((const GAS u4_a4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
__device__ __forceinline__ void move_run(T* __restrict__ dst, const T* __restrict__ src, int n,
                                         float s) {
  constexpr int per16 = 16 / sizeof(T);
  constexpr int kU = kChunkBytes / (16 * kBlock);  // 16-byte moves per thread per round
  static_assert(kU * 16 * kBlock == kChunkBytes, "a chunk's body is whole rounds of the workgroup");
  const bool one = s == 1.0f;
  const int tid = threadIdx.x;
  int head = (int)(((16 - ((uintptr_t)dst & 15)) & 15) / sizeof(T));
  if (head > n) head = n;
  if (tid < head) dst[tid] = scale_elem<T>(src[tid], s, one);
  const int body = (n - head) / per16;
  T* d = dst + head;
  const T* q = src + head;
  // rounds of kU words per thread (one round for a chunk of kChunkBytes),
  // each word predicated, so a thread's loads are all in flight together
  for (int u = tid; u < body; u += kU * kBlock) {
    uint4 w[kU];
#pragma unroll
    for (int j = 0; j < kU; ++j)
      if (u + j * kBlock < body) w[j] = load16(q + (size_t)(u + j * kBlock) * per16);
#pragma unroll
    for (int j = 0; j < kU; ++j) {
      if (u + j * kBlock < body) {
        const uint4 o = scale_vec<T>(w[j], s, one);
        __builtin_nontemporal_store(v4u{o.x, o.y, o.z, o.w}, (v4u*)(d + (size_t)(u + j * kBlock) * per16));
      }
    }
  }
  const int done = head + body * per16;
  const int tail = n - done;
  if (tid < tail) dst[done + tid] = scale_elem<T>(src[done + tid], s, one);
}

__global__ void __launch_bounds__(kBlock) bucket_kernel(const BucketArgs a) {
  const Chunk ch = a.chunks[blockIdx.x];
  char* tp = (char*)a.ptr[ch.t_slot];
  char* bp = (char*)a.ptr[ch.b_slot];
  if (a.dtype == DT_F32) {
    float* t = (float*)tp + ch.t_off;
    float* b = (float*)bp + ch.b_off;
    if (a.unpack) move_run<float>(t, b, ch.n, a.scale);
    else move_run<float>(b, t, ch.n, a.scale);
  } else {
    uint16_t* t = (uint16_t*)tp + ch.t_off;
    uint16_t* b = (uint16_t*)bp + ch.b_off;
    if (a.unpack) move_run<uint16_t>(t, b, ch.n, a.scale);
    else move_run<uint16_t>(b, t, ch.n, a.scale);
  }
}

// Plain copy of n16 16-byte words, streamed past the caches: each thread
// has kCopyUnroll loads in flight before it stores, and the grid gives each
// workgroup one span of kBlock * kCopyUnroll words (the fastest copy of the
// streaming probes below); the last partial round is predicated.
constexpr int kCopyUnroll = 8;
__global__ void __launch_bounds__(kBlock) copy_kernel(uint4* __restrict__ dst,
                                                      const uint4* __restrict__ src, size_t n16) {
  const size_t span = (size_t)kBlock * kCopyUnroll;
  const size_t step = (size_t)gridDim.x * span;
  size_t i = (size_t)blockIdx.x * span + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * kBlock < n16; i += step) {
    v4u v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load((const v4u*)(src + i + u * kBlock));
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], (v4u*)(dst + i + u * kBlock));
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u)
    if (i + u * kBlock < n16) dst[i + u * kBlock] = src[i + u * kBlock];
}

// Streaming-ceiling probes: the same 16-byte traffic as copy_kernel with
// the knobs that decide how close a kernel gets to peak HBM bandwidth --
// U loads in flight per thread, nontemporal (streaming) or ordinary
// accesses, and the grid (a grid-stride loop over a resident grid, or one
// workgroup per span of kBlock * U words).  KIND 0 copies, 1 only reads
// (each workgroup stores one word of XORed data so the loads stay live),
// 2 only writes.
template <int KIND, int U, bool NT>
__global__ void __launch_bounds__(kBlock) stream_kernel(uint4* __restrict__ dst,
                                                        const uint4* __restrict__ src, size_t n16) {
  const size_t span = (size_t)kBlock * U;
  const size_t step = (size_t)gridDim.x * span;
  size_t i = (size_t)blockIdx.x * span + threadIdx.x;
  v4u acc = {0u, 0u, 0u, 0u};
  const v4u fillv = {(unsigned)i, 1u, 2u, 3u};
  for (; i + (U - 1) * kBlock < n16; i += step) {
    v4u v[U];
    if (KIND != 2) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = NT ? __builtin_nontemporal_load((const v4u*)(src + i + u * kBlock))
                  : *(const v4u*)(src + i + u * kBlock);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (KIND == 1) {
        acc ^= v[u];
      } else {
        const v4u w = KIND == 2 ? fillv : v[u];
        if (NT) __builtin_nontemporal_store(w, (v4u*)(dst + i + u * kBlock));
        else *(v4u*)(dst + i + u * kBlock) = w;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (i + u * kBlock < n16) {
      if (KIND == 0) dst[i + u * kBlock] = src[i + u * kBlock];
      else if (KIND == 1) acc ^= *(const v4u*)(src + i + u * kBlock);
      else *(v4u*)(dst + i + u * kBlock) = fillv;
    }
  }
  if (KIND == 1) {
    // one word per workgroup: the XOR of the lanes' accumulators
    for (int m = 1; m < 64; m <<= 1) {
      acc.x ^= (unsigned)__shfl_xor((int)acc.x, m);
      acc.y ^= (unsigned)__shfl_xor((int)acc.y, m);
      acc.z ^= (unsigned)__shfl_xor((int)acc.z, m);
      acc.w ^= (unsigned)__shfl_xor((int)acc.w, m);
    }
    if (threadIdx.x == 0) *(v4u*)(dst + blockIdx.x) = acc;
  }
}

// ================================================================ host side
namespace {

struct DevInfo {
  int cus = 0;
  std::map<std::pair<int, int>, int> occ;  // (instance, lds bytes) -> resident workgroups per CU
};
std::mutex g_mu;
std::map<int, DevInfo> g_dev;

int device_cus(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& d = g_dev[dev];
  if (d.cus == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    d.cus = v;
  }
  return d.cus;
}

typedef void (*ExecFn)(const ExecArgs);
ExecFn exec_instance(int K, int NS, bool TR) {
  if (K != kWideK) return exec_kernel<1, kNS, false>;
  if (NS != 0) return exec_kernel<kWideK, kWideNS, false>;
  return TR ? exec_kernel<kWideK, 0, true> : exec_kernel<kWideK, 0, false>;
}

int exec_occupancy(int dev, int K, int NS, bool TR, int lds_bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& d = g_dev[dev];
  const std::pair<int, int> key(K * 16 + NS + (TR ? 256 : 0), lds_bytes);
  auto it = d.occ.find(key);
  if (it != d.occ.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, exec_instance(K, NS, TR), kBlock, lds_bytes) !=
          hipSuccess ||
      nb <= 0)
    nb = 2;
  d.occ[key] = nb;
  return nb;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GTF_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

namespace {
// As many workgroups as fit at once, spread so that every workgroup gets the
// same number of items (the last round is not left half empty).  A group
// that stages nothing per workgroup (no column or row values, one stage, no
// reduction) has nothing to share between the items of a workgroup: it
// gets one short-lived workgroup per item instead (measured on the
// one-launch epilogue of 194 gradients, 151M fp32 elements, into bucket
// slots: 384 -> 343 us; groups that stage values lose that way).
int launch_exec(const ExecArgs& a, int lds_bytes, hipStream_t stream) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const int64_t resident = (int64_t)device_cus(dev) * exec_occupancy(dev, a.K, a.NS, a.n_tr > 0, lds_bytes);
  const int64_t rounds = (a.n_items + resident - 1) / resident;
  int64_t grid = (a.n_items + rounds - 1) / rounds;
  const bool stages_nothing = a.n_col == 0 && a.n_stages == 1 && a.stage[0].row_len == 0 &&
                              a.stage[0].red == 0 && a.n_tr == 0;
  if (stages_nothing) grid = std::min<int64_t>(a.n_items, 0x7fffffff);
  hipLaunchKernelGGL(exec_instance(a.K, a.NS, a.n_tr > 0), dim3((unsigned)grid), dim3(kBlock), lds_bytes, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "exec_kernel launch");
  return GTF_OK;
}
}  // namespace

int launch_multi(const CompiledGroup& cg, const void* ws, size_t off_ptrs, size_t off_vec,
                 int64_t n_items, hipStream_t stream) {
  if (n_items == 0) return GTF_OK;
  ExecArgs a = cg.args;
  a.n_items = n_items;
  a.m_items = (const MultiItem*)ws;
  a.m_ptrs = (void* const*)((const char*)ws + off_ptrs);
  a.m_vec = (const uint32_t*)((const char*)ws + off_vec);
  a.n_slots = cg.n_slots;
  return launch_exec(a, cg.lds_bytes, stream);
}

int upload_bytes(void* dst, const void* src, size_t n, hipStream_t stream) {
  if (n == 0) return GTF_OK;
  hipError_t e = hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "table upload");
  return GTF_OK;
}

int launch_group(const CompiledGroup& cg, void* const* tensor_ptrs, hipStream_t stream) {
  ExecArgs a = cg.args;
  if (a.n_items == 0) return GTF_OK;
  bool any_reduce = false;
  for (int st = 0; st < a.n_stages; ++st)
    if (a.stage[st].red) any_reduce = true;
  if (a.C == 0 && !any_reduce) return GTF_OK;
  // per slot: 16-byte accesses (u8: 8-byte) need an aligned pointer and,
  // for [R,C] tensors of more than one row, rows a multiple of 8 elements
  const bool rows8 = a.R <= 1 || (a.C % kV) == 0;
  a.vec_slots = 0;
  for (int s = 0; s < cg.n_slots; ++s) {
    void* ptr = tensor_ptrs[cg.slot_tensor[s]];
    if (ptr == nullptr && cg.slot_numel[s] > 0)
      return fail(GTF_E_INVALID, "tensor " + std::to_string(cg.slot_tensor[s]) + " has no device pointer");
    a.ptr[s] = ptr;
    const uintptr_t align = cg.slot_dtype[s] == GTF_U8 ? 8 : 16;
    const bool contiguous = a.cstride[s] == 1 && (a.rstride[s] == 0 || rows8);
    if (contiguous && ((uintptr_t)ptr % align) == 0) a.vec_slots |= 1u << s;
  }
  // a staged bf16 transposed source reads 8 elements per load when its
  // pointer and row pitch keep those loads 16-byte aligned
  a.tr_vec = a.n_tr > 0 && a.tr_bf16 && ((uintptr_t)a.ptr[a.tr_slot] % 16) == 0 &&
             (a.cstride[a.tr_slot] % kV) == 0;
  a.m_items = nullptr;
  return launch_exec(a, cg.lds_bytes, stream);
}

namespace {
int launch_bucket_table(const BucketPlan& b, const Chunk* table, const void* const* tens, void* const* bk,
                        float scale, bool unpack, bool per_tensor, hipStream_t stream) {
  for (const BucketPlan::Launch& L : b.launches) {
    BucketArgs a;
    a.scale = scale;
    a.unpack = unpack ? 1 : 0;
    a.dtype = b.dtype == GTF_BF16 ? DT_BF16 : DT_F32;
    const int nt = L.t1 - L.t0;
    for (int k = 0; k < kMaxBucketPtrs; ++k) a.ptr[k] = nullptr;
    for (int i = 0; i < nt; ++i) {
      const void* p = tens[L.t0 + i];
      if (p == nullptr && b.numel[L.t0 + i] > 0)
        return fail(GTF_E_INVALID, "tensor " + std::to_string(L.t0 + i) + " pointer is NULL");
      a.ptr[i] = const_cast<void*>(p);
    }
    for (int k = L.b0; k <= L.b1; ++k) {
      if (bk[k] == nullptr && b.bucket_numel[k] > 0)
        return fail(GTF_E_INVALID, "bucket " + std::to_string(k) + " pointer is NULL");
      a.ptr[nt + (k - L.b0)] = bk[k];
    }
    if (!per_tensor) {
      const int64_t nch = L.c1 - L.c0;
      if (nch == 0) continue;
      a.chunks = table + L.c0;
      a.n_chunks = (int32_t)nch;
      hipLaunchKernelGGL(bucket_kernel, dim3((unsigned)nch), dim3(kBlock), 0, stream, a);
    } else {
      int64_t c = L.c0;
      while (c < L.c1) {
        int64_t e = c + 1;
        while (e < L.c1 && b.chunks[e].t_slot == b.chunks[c].t_slot) ++e;
        a.chunks = table + c;
        a.n_chunks = (int32_t)(e - c);
        hipLaunchKernelGGL(bucket_kernel, dim3((unsigned)(e - c)), dim3(kBlock), 0, stream, a);
        c = e;
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "bucket_kernel launch");
  }
  return GTF_OK;
}
}  // namespace

int launch_bucket(const BucketPlan& b, const void* const* tens, void* const* bk, float scale,
                  bool unpack, bool per_tensor, hipStream_t stream) {
  return launch_bucket_table(b, (const Chunk*)b.workspace, tens, bk, scale, unpack, per_tensor, stream);
}

// ---------------------------------------------------------------- allocation-free pack
// The chunk table of bucket_pack_static lives here, in device memory the
// library holds for the life of the process on each GPU it runs on, rather
// than in a workspace the caller allocates.  On the host, `scratch` only
// names the symbol: its device address is taken once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to a kernel or a copy.  Every call on one GPU shares the one
// array, so calls that overlap on a GPU race.
constexpr size_t kStaticChunkBytes = size_t(1) << 20;  // 43,690 chunks of <= 16 KiB
static __device__ __align__(256) unsigned char scratch[kStaticChunkBytes];

namespace {
std::map<int, void*> g_scratch;  // device -> address of its scratch (under g_mu)

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    it = g_scratch.emplace(dev, ptr).first;
  }
  *out = it->second;
  return GTF_OK;
}
}  // namespace

int launch_bucket_static(const BucketPlan& b, const void* const* tens, void* const* bk, float scale,
                         hipStream_t stream) {
  const size_t bytes = b.chunks.size() * sizeof(Chunk);
  if (bytes > kStaticChunkBytes)
    return fail(GTF_E_LIMIT, "chunk table of " + std::to_string(bytes) + " bytes exceeds the " +
                                 std::to_string(kStaticChunkBytes) + "-byte static scratch");
  void* table = nullptr;
  int st = scratch_address(&table);
  if (st != GTF_OK) return st;
  if (bytes > 0) {
    // a copy, not a memset: the table overwrites what an earlier call left
    hipError_t e = hipMemcpyAsync(table, b.chunks.data(), bytes, hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "chunk table upload to the static scratch");
  }
  return launch_bucket_table(b, (const Chunk*)table, tens, bk, scale, false, false, stream);
}

int upload_chunks(BucketPlan& b, void* ws, hipStream_t stream) {
  if (!b.chunks.empty()) {
    hipError_t e = hipMemcpyAsync(ws, b.chunks.data(), b.chunks.size() * sizeof(Chunk),
                                  hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "chunk table upload");
  }
  b.workspace = ws;
  return GTF_OK;
}

namespace {
typedef void (*StreamFn)(uint4*, const uint4*, size_t);
template <int KIND>
StreamFn stream_instance(int depth, bool nt) {
  switch (depth) {
    case 4: return nt ? stream_kernel<KIND, 4, true> : stream_kernel<KIND, 4, false>;
    case 8: return nt ? stream_kernel<KIND, 8, true> : stream_kernel<KIND, 8, false>;
    case 16: return nt ? stream_kernel<KIND, 16, true> : stream_kernel<KIND, 16, false>;
    default: return nullptr;
  }
}
}  // namespace

int launch_stream_probe(int kind, int depth, int nontemporal, int grid_per_cu, void* dst,
                        const void* src, size_t nbytes, hipStream_t stream) {
  StreamFn fn = kind == 0   ? stream_instance<0>(depth, nontemporal != 0)
                : kind == 1 ? stream_instance<1>(depth, nontemporal != 0)
                : kind == 2 ? stream_instance<2>(depth, nontemporal != 0)
                            : nullptr;
  if (fn == nullptr) return fail(GTF_E_INVALID, "stream probe: kind 0..2 and depth 4, 8 or 16");
  if (grid_per_cu < 0) return fail(GTF_E_INVALID, "stream probe: grid_per_cu < 0");
  const size_t n16 = nbytes / 16;
  if (n16 == 0) return GTF_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  size_t grid = (n16 + (size_t)kBlock * depth - 1) / ((size_t)kBlock * depth);
  if (grid_per_cu > 0) grid = std::min(grid, (size_t)device_cus(dev) * (size_t)grid_per_cu);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(kBlock), 0, stream, (uint4*)dst, (const uint4*)src, n16);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "stream_kernel launch");
  return GTF_OK;
}

int launch_copy(void* dst, const void* src, size_t nbytes, hipStream_t stream) {
  const size_t n16 = nbytes / 16;
  if (n16 == 0) return GTF_OK;
  size_t grid = (n16 + (size_t)kBlock * kCopyUnroll - 1) / ((size_t)kBlock * kCopyUnroll);
  if (grid > 0x7fffffffu) grid = 0x7fffffffu;  // the kernel's loop covers the rest
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, (uint4*)dst,
                     (const uint4*)src, n16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "copy_kernel launch");
  return GTF_OK;
}

}  // namespace gtf
