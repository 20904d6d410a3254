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

#include <map>
#include <mutex>
#include <string>

#include "gtf.h"
#include "isa.h"
#include "plan.h"

namespace gtf {

enum Mode { M_ELEM = 0, M_ROW = 1, M_COL = 2 };

// ---------------------------------------------------------------- numerics
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  // fp32 -> bf16 round to nearest even (one v_cvt_pk_bf16_f32 on gfx950)
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}

__device__ __forceinline__ float f_sigmoid(float x) {
  // 1 / (1 + e^-x), written as e^x / (1 + e^x) for x < 0 so the tail keeps
  // its relative accuracy; one correctly rounded division
  const float e = expf(-fabsf(x));
  const float num = x >= 0.f ? 1.f : e;
  return num / (1.f + e);
}
__device__ __forceinline__ float f_gelu(float x) {
  // x/2 * erfc(-x/sqrt(2)): the erfc form keeps the negative tail accurate.
  // The fp32 argument a = -x/sqrt(2) carries a rounding error a_lo that
  // erfc's slope magnifies by about 2a^2 in relative terms (1e-6 near
  // x = -5).  a_lo is recovered exactly with one fma and a split constant,
  // and erfc(a_hi + a_lo) = erfc(a_hi) * (1 - L(a_hi) * a_lo) to first
  // order, where L = 2 exp(-a^2) / (sqrt(pi) erfc(a)) is erfc's negative
  // log-derivative.  The Mills-ratio bounds bracket L between
  // a + sqrt(a^2 + 4/pi) and a + sqrt(a^2 + 2); the lower one is used (for
  // a < 0 it overestimates a term that is below 1e-7 anyway).
  const float c_hi = -0.70710678118654752440f;               // -1/sqrt(2) in fp32
  const float c_lo = -1.21016170e-08f;                       // -1/sqrt(2) - c_hi
  const float a_hi = x * c_hi;
  const float a_lo = __builtin_fmaf(x, c_hi, -a_hi) + x * c_lo;
  const float L = a_hi + __builtin_amdgcn_sqrtf(a_hi * a_hi + 1.27323954473516268615f);  // 4/pi
  const float e = erfcf(a_hi);
  return (0.5f * x) * (e - e * (L * a_lo));
}
__device__ __forceinline__ float f_relu(float x) { return x > 0.f ? x : 0.f; }

// tanh without a lane-dependent branch (a branch inside an interpreter case
// would make the compiler linearise the whole dispatch switch): both forms
// are computed and one is selected.  |x| < 0.625: x + x^3 P(x^2), with P of
// degree 4 fitted here by weighted least squares on Chebyshev nodes (max
// relative error 7.4e-8 in fp32); otherwise 1 - 2 / (e^{2|x|} + 1), which
// has no cancellation there (the result is at least 0.55).
__device__ __forceinline__ float f_tanh(float x) {
  const float ax = fabsf(x);
  const float u = ax * ax;
  float p = -5.691985599696636e-03f;
  p = __builtin_fmaf(p, u, 2.0626291632652283e-02f);
  p = __builtin_fmaf(p, u, -5.373531952500343e-02f);
  p = __builtin_fmaf(p, u, 1.3331381976604462e-01f);
  p = __builtin_fmaf(p, u, -3.333328068256378e-01f);
  const float small = __builtin_fmaf(ax * u, p, ax);
  const float e = expf(2.0f * ax);
  const float big = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  return copysignf(ax < 0.625f ? small : big, x);
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

// ---------------------------------------------------------------- context
struct Tile {
  int64_t row;   // global row
  int64_t col;   // global column of the first element
  int64_t eoff;  // element offset of the tile in [R,C] tensors
  int cl;        // column inside the staged panel
  int rr;        // row inside the row block
  int cnt;       // valid elements in the tile
  bool valid;    // the tile exists (row and column in range)
  bool vec;      // whole tile, 16-byte aligned: vector path
  const char* ring;  // this tile's stage of the wave's LDS ring (or null)
  int lane;      // lane within the wave
};

template <int V, int MODE>
__device__ __forceinline__ int64_t elem_offset(const ExecArgs& a, int slot, const Tile& t) {
  if (MODE == M_ELEM) return t.eoff;
  if (MODE == M_ROW) return t.row * a.rstride[slot];
  return t.col * a.cstride[slot];
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void load_f32(float (&d)[V], const ExecArgs& a, int slot, const Tile& t,
                                         int ring_off) {
  if (MODE == M_ELEM && V == 8) {
    if ((FAST || t.vec) && t.ring != nullptr && ring_off >= 0) {
      const char* q = t.ring + ring_off + t.lane * 16;
      const float4 x = *(const float4*)q;
      const float4 y = *(const float4*)(q + 1024);
      d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
      d[4] = y.x; d[5] = y.y; d[6] = y.z; d[7] = y.w;
      return;
    }
  }
  const float* p = (const float*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (FAST || t.vec) {
      const float4 x = *(const float4*)p;
      const float4 y = *(const float4*)(p + 4);
      d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
      d[4] = y.x; d[5] = y.y; d[6] = y.z; d[7] = y.w;
      return;
    }
  }
  if (MODE == M_ELEM) {  // partial tile: clamped in-bounds reads, no branch
    const float* b = (const float*)a.ptr[slot];
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = b[(t.valid && i < t.cnt) ? t.eoff + i : 0];
    return;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = p[i];
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void load_bf16(float (&d)[V], const ExecArgs& a, int slot, const Tile& t,
                                         int ring_off) {
  if (MODE == M_ELEM && V == 8) {
    if ((FAST || t.vec) && t.ring != nullptr && ring_off >= 0) {
      const uint4 w = *(const uint4*)(t.ring + ring_off + t.lane * 16);
      d[0] = bf16_lo(w.x); d[1] = bf16_hi(w.x); d[2] = bf16_lo(w.y); d[3] = bf16_hi(w.y);
      d[4] = bf16_lo(w.z); d[5] = bf16_hi(w.z); d[6] = bf16_lo(w.w); d[7] = bf16_hi(w.w);
      return;
    }
  }
  const uint16_t* p = (const uint16_t*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (FAST || t.vec) {
      const uint4 w = *(const uint4*)p;
      d[0] = bf16_lo(w.x); d[1] = bf16_hi(w.x); d[2] = bf16_lo(w.y); d[3] = bf16_hi(w.y);
      d[4] = bf16_lo(w.z); d[5] = bf16_hi(w.z); d[6] = bf16_lo(w.w); d[7] = bf16_hi(w.w);
      return;
    }
  }
  if (MODE == M_ELEM) {
    const uint16_t* b = (const uint16_t*)a.ptr[slot];
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = bf16_at(b + ((t.valid && i < t.cnt) ? t.eoff + i : 0));
    return;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = bf16_at(p + i);
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void load_u8(float (&d)[V], const ExecArgs& a, int slot, const Tile& t,
                                         int ring_off) {
  if (MODE == M_ELEM && V == 8) {
    if ((FAST || t.vec) && t.ring != nullptr && ring_off >= 0) {
      const char* q = t.ring + ring_off + t.lane * 4;
      const uint32_t w0 = *(const uint32_t*)q;
      const uint32_t w1 = *(const uint32_t*)(q + 256);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = (float)((w0 >> (8 * i)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[4 + i] = (float)((w1 >> (8 * i)) & 0xFFu);
      return;
    }
  }
  const uint8_t* p = (const uint8_t*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (FAST || t.vec) {
      const uint2 w = *(const uint2*)p;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = (float)((w.x >> (8 * i)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[4 + i] = (float)((w.y >> (8 * i)) & 0xFFu);
      return;
    }
  }
  if (MODE == M_ELEM) {
    const uint8_t* b = (const uint8_t*)a.ptr[slot];
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = (float)b[(t.valid && i < t.cnt) ? t.eoff + i : 0];
    return;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = (float)p[i];
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void store_f32(const float (&s)[V], const ExecArgs& a, int slot, const Tile& t) {
  float* p = (float*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (FAST || t.vec) {
      *(float4*)p = make_float4(s[0], s[1], s[2], s[3]);
      *(float4*)(p + 4) = make_float4(s[4], s[5], s[6], s[7]);
      return;
    }
  }
  if (MODE == M_ELEM) {  // partial tile: one predicated store per element
    float* b = (float*)a.ptr[slot];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool on = t.valid && i < t.cnt;
      pstore_b32(b + (on ? t.eoff + i : 0), __float_as_uint(s[i]), lanes(on));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) p[i] = s[i];
}

template <int V, int MODE, bool FAST>
__device__ __forceinline__ void store_bf16(const float (&s)[V], const ExecArgs& a, int slot, const Tile& t) {
  uint16_t* p = (uint16_t*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (FAST || t.vec) {
      *(uint4*)p = make_uint4(pack_bf16(s[0], s[1]), pack_bf16(s[2], s[3]),
                              pack_bf16(s[4], s[5]), pack_bf16(s[6], s[7]));
      return;
    }
  }
  if (MODE == M_ELEM) {
    uint16_t* b = (uint16_t*)a.ptr[slot];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const bool on = t.valid && i < t.cnt;
      pstore_b16(b + (on ? t.eoff + i : 0), pack_bf16(s[i], 0.f) & 0xFFFFu, lanes(on));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) p[i] = (uint16_t)(pack_bf16(s[i], 0.f) & 0xFFFFu);
}

// ---------------------------------------------------------------- ops
template <int V, int F>
__device__ __forceinline__ void unary(float (&r)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float x = r[i];
    float y;
    if (F == F_EXP) y = expf(x);
    else if (F == F_TANH) y = f_tanh(x);
    else if (F == F_SIGMOID) y = f_sigmoid(x);
    else if (F == F_RELU) y = f_relu(x);
    else if (F == F_GELU) y = f_gelu(x);
    else if (F == F_SQUARE) y = x * x;
    else if (F == F_SQRT) y = sqrtf(x);
    else if (F == F_RECIP) y = 1.0f / x;
    else y = -x;  // F_NEG
    r[i] = y;
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

// x: V consecutive fp32 values in LDS (32-byte aligned for V == 8)
template <int V>
__device__ __forceinline__ void lds_vec(float (&d)[V], const float* x) {
  if (V == 8) {
    const float4 u = *(const float4*)x;
    const float4 w = *(const float4*)(x + 4);
    const float xs[8] = {u.x, u.y, u.z, u.w, w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = xs[i % 8];
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) d[i] = x[i];
  }
}

template <int V, int OP>
__device__ __forceinline__ void xvec(float (&r)[V], const float* x) {
  float xs[V];
  lds_vec<V>(xs, x);
#pragma unroll
  for (int i = 0; i < V; ++i) r[i] = xop<OP>(r[i], xs[i]);
}

template <int V, int OP>
__device__ __forceinline__ void xscalar(float (&r)[V], float x) {
#pragma unroll
  for (int i = 0; i < V; ++i) r[i] = xop<OP>(r[i], x);
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
// A, B and the spill slots hold one tile each.  The next instruction word is
// fetched while the current one executes.  FAST is the instance for tiles
// that are whole, in range and vector-aligned in every lane of the wave: it
// has no lane-dependent branch, so the compiler keeps the dispatch switch a
// tree of scalar branches (a lane-dependent branch anywhere in the loop
// makes it linearise the switch into a chain of guarded blocks).  The other
// instance handles partial tiles at row and tensor ends.
template <int V, int MODE, bool FAST>
__device__ __forceinline__ void interpret(const ExecArgs& a, const Instr* prog, int n,
                                          const Tile& t, float* lds_col, float* lds_row,
                                          float& acc, bool store_global) {
  float A[V], B[V], S0[V], S1[V], S2[V], S3[V], S4[V], S5[V];
  if (n <= 0) return;
  Instr cur = prog[0];
  for (int pc = 0; pc < n; ++pc) {
    const Instr nxt = prog[pc + 1 < n ? pc + 1 : pc];
    const int arg = cur.arg;
    const float* col = lds_col + arg * a.PW + t.cl;
    switch (cur.code) {
      case F_LD_F32_A: load_f32<V, MODE, FAST>(A, a, arg, t, __float_as_int(cur.imm)); break;
      case F_LD_BF16_A: load_bf16<V, MODE, FAST>(A, a, arg, t, __float_as_int(cur.imm)); break;
      case F_LD_U8_A: load_u8<V, MODE, FAST>(A, a, arg, t, __float_as_int(cur.imm)); break;
      case F_LD_F32_B: load_f32<V, MODE, FAST>(B, a, arg, t, __float_as_int(cur.imm)); break;
      case F_LD_BF16_B: load_bf16<V, MODE, FAST>(B, a, arg, t, __float_as_int(cur.imm)); break;
      case F_LD_U8_B: load_u8<V, MODE, FAST>(B, a, arg, t, __float_as_int(cur.imm)); break;
      case F_COL_A: if (MODE == M_ELEM) lds_vec<V>(A, col); break;
      case F_ROW_A: if (MODE == M_ELEM) fill<V>(A, lds_row[arg * a.RB + t.rr]); break;
      case F_IMM_A: fill<V>(A, cur.imm); break;
      case F_COL_B: if (MODE == M_ELEM) lds_vec<V>(B, col); break;
      case F_ROW_B: if (MODE == M_ELEM) fill<V>(B, lds_row[arg * a.RB + t.rr]); break;
      case F_IMM_B: fill<V>(B, cur.imm); break;
      case F_A2B: copy<V>(B, A); break;
      case F_B2A: copy<V>(A, B); break;
      case F_A2S0: copy<V>(S0, A); break;
      case F_A2S1: copy<V>(S1, A); break;
      case F_A2S2: copy<V>(S2, A); break;
      case F_A2S3: copy<V>(S3, A); break;
      case F_A2S4: copy<V>(S4, A); break;
      case F_A2S5: copy<V>(S5, A); break;
      case F_B2S0: copy<V>(S0, B); break;
      case F_B2S1: copy<V>(S1, B); break;
      case F_B2S2: copy<V>(S2, B); break;
      case F_B2S3: copy<V>(S3, B); break;
      case F_B2S4: copy<V>(S4, B); break;
      case F_B2S5: copy<V>(S5, B); break;
      case F_S02A: copy<V>(A, S0); break;
      case F_S12A: copy<V>(A, S1); break;
      case F_S22A: copy<V>(A, S2); break;
      case F_S32A: copy<V>(A, S3); break;
      case F_S42A: copy<V>(A, S4); break;
      case F_S52A: copy<V>(A, S5); break;
      case F_S02B: copy<V>(B, S0); break;
      case F_S12B: copy<V>(B, S1); break;
      case F_S22B: copy<V>(B, S2); break;
      case F_S32B: copy<V>(B, S3); break;
      case F_S42B: copy<V>(B, S4); break;
      case F_S52B: copy<V>(B, S5); break;
      case F_EXP: unary<V, F_EXP>(A); break;
      case F_TANH: unary<V, F_TANH>(A); break;
      case F_SIGMOID: unary<V, F_SIGMOID>(A); break;
      case F_RELU: unary<V, F_RELU>(A); break;
      case F_GELU: unary<V, F_GELU>(A); break;
      case F_SQUARE: unary<V, F_SQUARE>(A); break;
      case F_SQRT: unary<V, F_SQRT>(A); break;
      case F_RECIP: unary<V, F_RECIP>(A); break;
      case F_NEG: unary<V, F_NEG>(A); break;
#define GTF_BIN(NAME, OP)                                                               \
  case F_##NAME: binop<V, OP>(A, B); break;                                             \
  case F_##NAME##_C: if (MODE == M_ELEM) xvec<V, OP>(A, col); break;                  \
  case F_##NAME##_R: if (MODE == M_ELEM) xscalar<V, OP>(A, lds_row[arg * a.RB + t.rr]); break; \
  case F_##NAME##_I: xscalar<V, OP>(A, cur.imm); break;
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
          for (int i = 0; i < V; ++i) acc += (FAST || (t.valid && i < t.cnt)) ? A[i] : 0.f;
        }
        break;
      case F_ST_LDS:
        if (MODE == M_ROW) lds_row[arg * a.RB + t.rr] = A[0];
        if (MODE == M_COL) lds_col[arg * a.PW + t.cl] = A[0];
        break;
      default:
        break;
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------- reduce tail
__device__ __forceinline__ float dpp_add(float v, int ctrl_id) {
  int x = __float_as_int(v);
  int y;
  switch (ctrl_id) {
    case 0: y = __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false); break;   // quad_perm [1,0,3,2]
    case 1: y = __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false); break;   // quad_perm [2,3,0,1]
    case 2: y = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
    default: y = __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false); break; // row_mirror
  }
  return v + __int_as_float(y);
}

// Sum over aligned segments of `width` lanes (a power of two <= 64); every
// lane of a segment ends with the segment's sum.
__device__ __forceinline__ float segment_sum(float v, int width) {
  if (width >= 2) v = dpp_add(v, 0);
  if (width >= 4) v = dpp_add(v, 1);
  if (width >= 8) v = dpp_add(v, 2);
  if (width >= 16) v = dpp_add(v, 3);
  if (width >= 32) v += __shfl_xor(v, 16);
  if (width >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Row result of the reduce tail, written by the lanes in `on` (one lane per
// row) with a predicated store.
__device__ __forceinline__ void store_reduced(const ExecArgs& a, int64_t row, float s, bool on) {
  const float v = a.reduce == 2 ? s / (float)a.C : s;
  const int slot = a.red_slot;
  const int64_t off = on ? row * a.rstride[slot] : 0;
  const uint64_t m = lanes(on);
  if (a.red_dtype == DT_BF16)
    pstore_b16((uint16_t*)a.ptr[slot] + off, pack_bf16(v, 0.f) & 0xFFFFu, m);
  else
    pstore_b32((float*)a.ptr[slot] + off, __float_as_uint(v), m);
}

// ---------------------------------------------------------------- LDS ring
// Direct global -> LDS loads (gfx950 global_load_lds): lane i's bytes land
// at M0 + i * size.  They are issued in inline assembly so the compiler does
// not treat every later LDS read as a possible alias of an in-flight copy
// (which would make it drain all of them); the kernel counts them itself
// and waits with an explicit vmcnt.  Neither asm clobbers memory, so the
// compiler keeps kernel arguments in registers across them; instead the
// ring pointer passes through the wait as an operand, which orders every
// ring read after the wait.  A stage is rewritten only one iteration after
// its reads, across the loop's back edge.  M0 is saved and restored.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(lds));
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  uint32_t save;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(save)
      : "v"(g), "s"(lds));
}

// Wait until at most n vector-memory operations of this wave are in flight
// (they complete in issue order; n <= 63).  Returns `ring` through the asm
// so reads through the result cannot move above the wait.
__device__ __forceinline__ const char* wait_vmcnt(int n, const char* ring) {
  switch (n) {
#define GTF_W(N) case N: asm volatile("s_waitcnt vmcnt(" #N ")" : "+s"(ring)); break;
    GTF_W(0) GTF_W(1) GTF_W(2) GTF_W(3) GTF_W(4) GTF_W(5) GTF_W(6) GTF_W(7)
    GTF_W(8) GTF_W(9) GTF_W(10) GTF_W(11) GTF_W(12) GTF_W(13) GTF_W(14) GTF_W(15)
    GTF_W(16) GTF_W(17) GTF_W(18) GTF_W(19) GTF_W(20) GTF_W(21) GTF_W(22) GTF_W(23)
    GTF_W(24) GTF_W(25) GTF_W(26) GTF_W(27) GTF_W(28) GTF_W(29) GTF_W(30) GTF_W(31)
    GTF_W(32) GTF_W(33) GTF_W(34) GTF_W(35) GTF_W(36) GTF_W(37) GTF_W(38) GTF_W(39)
    GTF_W(40) GTF_W(41) GTF_W(42) GTF_W(43) GTF_W(44) GTF_W(45) GTF_W(46) GTF_W(47)
    GTF_W(48) GTF_W(49) GTF_W(50) GTF_W(51) GTF_W(52) GTF_W(53) GTF_W(54) GTF_W(55)
    GTF_W(56) GTF_W(57) GTF_W(58) GTF_W(59) GTF_W(60) GTF_W(61) GTF_W(62)
#undef GTF_W
    default: asm volatile("s_waitcnt vmcnt(63)" : "+s"(ring)); break;
  }
  return ring;
}

// The pipelined inputs of a launch, read once from the kernel arguments.
struct RingInputs {
  const char* base[kMaxPipe];
  uint32_t off[kMaxPipe];
  int dt[kMaxPipe];
  int n;
};

// Issue the loads of one tile of every pipelined input into one ring
// stage.  All lanes take part; a lane whose tile is not a whole in-range
// tile loads the tensor's first tile instead (never read).
__device__ __forceinline__ void ring_issue(const RingInputs& in, uint32_t stage_lds, bool ok,
                                           int64_t eoff) {
  const int64_t off = ok ? eoff : 0;
#pragma unroll
  for (int k = 0; k < kMaxPipe; ++k) {
    if (k >= in.n) break;
    const uint32_t dst = stage_lds + in.off[k];
    if (in.dt[k] == DT_BF16) {
      dma16(in.base[k] + off * 2, dst);
    } else if (in.dt[k] == DT_F32) {
      const char* g = in.base[k] + off * 4;
      dma16(g, dst);
      dma16(g + 16, dst + 1024);
    } else {
      const char* g = in.base[k] + off;
      dma4(g, dst);
      dma4(g + 4, dst + 256);
    }
  }
}

// ---------------------------------------------------------------- executor
__global__ void __launch_bounds__(kBlock) exec_kernel(const ExecArgs a) {
  extern __shared__ float lds[];
  float* lds_col = lds;
  float* lds_row = lds + a.n_col_slots * a.PW;
  float* lds_red = lds_row + a.n_row_slots * a.RB;
  const int tid = threadIdx.x;
  const int tpr = 1 << a.tpr_log2;
  const int rpp = kBlock >> a.tpr_log2;
  const int sub = tid >> a.tpr_log2;
  const int lt = tid & (tpr - 1);
  const Instr* col_prog = a.prog;
  const Instr* row_prog = a.prog + a.n_col;
  const Instr* el_prog = a.prog + a.n_col + a.n_row;
  const int64_t erow_stride = a.R == 1 ? 0 : a.C;
  bool staged = false;
  float dummy = 0.f;
  const int lane = tid & 63;
  // the ring needs a whole first tile in every pipelined tensor (the
  // fallback address of out-of-range tiles)
  const bool ring_on = a.n_pipe > 0 && a.n_stage >= 2 && a.vec_ok && a.C >= kV && a.R >= 1;
  const bool vec_ok = a.vec_ok != 0;
  const int n_stage = ring_on ? a.n_stage : 1;
  const int ring_wait = (a.n_stage - 1) * a.n_dma;
  RingInputs rin;
  rin.n = ring_on ? a.n_pipe : 0;
#pragma unroll
  for (int k = 0; k < kMaxPipe; ++k) {
    const int slot = k < a.n_pipe ? a.pipe_slot[k] : 0;
    rin.base[k] = (const char*)a.ptr[slot];
    rin.off[k] = k < a.n_pipe ? (uint32_t)a.ring_off[slot] : 0u;
    rin.dt[k] = a.pipe_dt[k];
  }
  // this wave's ring: generic pointer for reads, LDS address for the loads
  const uint32_t wave = __builtin_amdgcn_readfirstlane((uint32_t)tid >> 6);
  const int ring_wave_off = a.ring_lds_off + (int)wave * a.n_stage * a.stage_bytes;
  const char* ring_gen = (const char*)lds + ring_wave_off;
  const uint32_t ring_w =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)((char*)lds) + (uint32_t)ring_wave_off;

  for (int64_t item = blockIdx.x; item < a.n_items; item += gridDim.x) {
    const int64_t rb = item / a.n_panels;
    const int p = (int)(item - rb * a.n_panels);
    const int64_t r0 = rb * a.RB;
    const int nr = (int)min((int64_t)a.RB, a.R - r0);
    const int64_t c0 = (int64_t)p * a.PW;
    const int nc = (int)min((int64_t)a.PW, a.C - c0);

    if (a.n_col > 0 && (a.n_panels > 1 || !staged)) {
      __syncthreads();
      for (int c = tid; c < nc; c += kBlock) {
        Tile t{0, c0 + c, 0, c, 0, 1, false};
        interpret<1, M_COL, false>(a, col_prog, a.n_col, t, lds_col, lds_row, dummy, rb == 0);
      }
      __syncthreads();
      staged = true;
    }
    if (a.n_row > 0) {
      __syncthreads();
      for (int r = tid; r < nr; r += kBlock) {
        Tile t{r0 + r, 0, 0, 0, r, 1, false};
        interpret<1, M_ROW, false>(a, row_prog, a.n_row, t, lds_col, lds_row, dummy, p == 0);
      }
      __syncthreads();
    }

    // element phase: each lane walks its tiles q = (pass, j) in order; the
    // pipelined inputs of tile q + n_stage - 1 are requested while tile q
    // is interpreted.  Cursors advance by increments (no divisions).
    const int npass = (nr + rpp - 1) / rpp;
    const int tpl = max(1, (nc + tpr * kV - 1) / (tpr * kV));  // tiles per lane per row
    const int nq = npass * tpl;
    int ip = 0, ij = 0, is = 0;  // issue cursor: pass, tile in row, stage
    auto issue_next = [&]() {
      const int rr = ip * rpp + sub;
      const int cl = (lt + ij * tpr) * kV;
      const bool ok = rr < nr && cl + kV <= nc;
      ring_issue(rin, ring_w + (uint32_t)(is * a.stage_bytes), ok, (r0 + rr) * erow_stride + c0 + cl);
      if (++ij == tpl) {
        ij = 0;
        ++ip;
      }
      if (++is == n_stage) is = 0;
    };
    if (ring_on) {
      const int pre = min(n_stage - 1, nq);
      for (int q = 0; q < pre; ++q) issue_next();
    }
    float acc = 0.f;
    int pass = 0, j = 0, stage = 0;
    for (int q = 0; q < nq; ++q) {
      const char* ring = nullptr;
      if (ring_on) {
        if (q + n_stage - 1 < nq) {
          issue_next();
          ring = wait_vmcnt(ring_wait, ring_gen);
        } else {
          ring = wait_vmcnt(0, ring_gen);
        }
      }
      const int rr = pass * rpp + sub;
      const int cl = (lt + j * tpr) * kV;
      const bool valid = rr < nr && cl < nc;
      Tile t;
      t.valid = valid;
      t.row = r0 + rr;
      t.col = c0 + cl;
      t.eoff = t.row * erow_stride + t.col;
      t.cl = cl;
      t.rr = rr;
      t.cnt = min(kV, nc - cl);
      t.vec = vec_ok && valid && t.cnt == kV;
      t.ring = ring_on ? ring + stage * a.stage_bytes : nullptr;
      t.lane = lane;
      // both branches are wave-uniform
      if (__all(t.vec)) {
        interpret<kV, M_ELEM, true>(a, el_prog, a.n_elem, t, lds_col, lds_row, acc, true);
      } else if (__any(valid)) {
        interpret<kV, M_ELEM, false>(a, el_prog, a.n_elem, t, lds_col, lds_row, acc, true);
      }
      if (a.reduce && j == tpl - 1) {
        const int w = min(tpr, 64);
        float s = segment_sum(acc, w);
        acc = 0.f;
        if (tpr <= 64) {
          store_reduced(a, r0 + rr, s, lt == 0 && rr < nr);
        } else {
          // rows wider than a wave: combine the per-wave sums through LDS in
          // a fixed order (every lane of a wave holds the same sum and
          // writes it; every lane reads the totals of its own row)
          const int wpr = tpr >> 6;        // waves per row
          lds_red[tid >> 6] = s;
          __syncthreads();
          float tot = 0.f;
          for (int k = 0; k < wpr; ++k) tot += lds_red[sub * wpr + k];
          store_reduced(a, r0 + rr, tot, lt == 0 && rr < nr);
          __syncthreads();
        }
      }
      if (++j == tpl) {
        j = 0;
        ++pass;
      }
      if (++stage == n_stage) stage = 0;
    }
  }
}

// ---------------------------------------------------------------- buckets
// One workgroup per chunk: a run of up to kChunkElems elements of one tensor
// copied to or from its place in its bucket, times the scale.  The side that
// lives in the bucket is usually not 16-byte aligned (offsets are dense), so
// a few head elements bring the destination to a 16-byte boundary, the body
// moves 16 bytes per lane per step, and a tail finishes.
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

template <typename T>
__device__ __forceinline__ void move_run(T* __restrict__ dst, const T* __restrict__ src, int n,
                                         float s) {
  constexpr int per16 = 16 / sizeof(T);
  const bool one = s == 1.0f;
  const int tid = threadIdx.x;
  int head = (int)(((16 - ((uintptr_t)dst & 15)) & 15) / sizeof(T));
  if (head > n) head = n;
  if (tid < head) dst[tid] = scale_elem<T>(src[tid], s, one);
  const int body = (n - head) / per16;
  T* d = dst + head;
  const T* q = src + head;
  for (int u = tid; u < body; u += kBlock) {
    uint4 w;
    __builtin_memcpy(&w, q + (size_t)u * per16, 16);  // source may be 4-byte aligned
    *(uint4*)(d + (size_t)u * per16) = scale_vec<T>(w, s, one);
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

__global__ void __launch_bounds__(kBlock) copy_kernel(uint4* __restrict__ dst,
                                                      const uint4* __restrict__ src, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += (size_t)gridDim.x * kBlock)
    dst[i] = src[i];
}

// ================================================================ host side
namespace {

struct DevInfo {
  int cus = 0;
  std::map<int, int> occ;  // lds bytes -> resident workgroups per CU
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

int exec_occupancy(int dev, int lds_bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  DevInfo& d = g_dev[dev];
  auto it = d.occ.find(lds_bytes);
  if (it != d.occ.end()) return it->second;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, exec_kernel, kBlock, lds_bytes) != hipSuccess ||
      nb <= 0)
    nb = 2;
  d.occ[lds_bytes] = nb;
  return nb;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(GTF_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

int launch_group(const CompiledGroup& cg, void* const* tensor_ptrs, hipStream_t stream) {
  ExecArgs a = cg.args;
  if (a.n_items == 0) return GTF_OK;
  if (a.C == 0 && a.reduce == 0) return GTF_OK;
  bool vec = true;
  for (int s = 0; s < cg.n_slots; ++s) {
    void* ptr = tensor_ptrs[cg.slot_tensor[s]];
    if (ptr == nullptr && cg.slot_numel[s] > 0)
      return fail(GTF_E_INVALID, "tensor " + std::to_string(cg.slot_tensor[s]) + " has no device pointer");
    a.ptr[s] = ptr;
    if (((uintptr_t)ptr & 15) != 0) vec = false;
  }
  if (a.R > 1 && (a.C % kV) != 0) vec = false;
  a.vec_ok = vec ? 1 : 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const int64_t resident = (int64_t)device_cus(dev) * exec_occupancy(dev, cg.lds_bytes);
  const int64_t grid = a.n_items < resident ? a.n_items : resident;
  hipLaunchKernelGGL(exec_kernel, dim3((unsigned)grid), dim3(kBlock), cg.lds_bytes, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "exec_kernel launch");
  return GTF_OK;
}

int launch_bucket(const BucketPlan& b, const void* const* tens, void* const* bk, float scale,
                  bool unpack, bool per_tensor, hipStream_t stream) {
  const Chunk* table = (const Chunk*)b.workspace;
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

int upload_chunks(BucketPlan& b, void* ws, hipStream_t stream) {
  if (!b.chunks.empty()) {
    hipError_t e = hipMemcpyAsync(ws, b.chunks.data(), b.chunks.size() * sizeof(Chunk),
                                  hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "chunk table upload");
  }
  b.workspace = ws;
  return GTF_OK;
}

int launch_copy(void* dst, const void* src, size_t nbytes, hipStream_t stream) {
  const size_t n16 = nbytes / 16;
  if (n16 == 0) return GTF_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  size_t grid = (n16 + kBlock - 1) / kBlock;
  const size_t cap = (size_t)device_cus(dev) * 8;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(kBlock), 0, stream, (uint4*)dst,
                     (const uint4*)src, n16);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "copy_kernel launch");
  return GTF_OK;
}

}  // namespace gtf
