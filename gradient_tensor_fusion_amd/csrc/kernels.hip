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
// load from the kernarg segment and a scalar branch tree); every register
// index is a compile-time constant of its case, so the stack stays in
// VGPRs.
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
  const float L = a_hi + sqrtf(a_hi * a_hi + 1.27323954473516268615f);  // 4/pi
  const float e = erfcf(a_hi);
  return (0.5f * x) * (e - e * (L * a_lo));
}
__device__ __forceinline__ float f_relu(float x) { return x > 0.f ? x : 0.f; }

// ---------------------------------------------------------------- context
struct Tile {
  int64_t row;   // global row
  int64_t col;   // global column of the first element
  int64_t eoff;  // element offset of the tile in [R,C] tensors
  int cl;        // column inside the staged panel
  int rr;        // row inside the row block
  int cnt;       // valid elements in the tile
  bool vec;      // whole tile, 16-byte aligned: vector path
};

template <int V, int MODE>
__device__ __forceinline__ int64_t elem_offset(const ExecArgs& a, int slot, const Tile& t) {
  if (MODE == M_ELEM) return t.eoff;
  if (MODE == M_ROW) return t.row * a.rstride[slot];
  return t.col * a.cstride[slot];
}

template <int V, int MODE>
__device__ __forceinline__ void load_f32(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const float* p = (const float*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (t.vec) {
      const float4 x = *(const float4*)p;
      const float4 y = *(const float4*)(p + 4);
      d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
      d[4] = y.x; d[5] = y.y; d[6] = y.z; d[7] = y.w;
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = (i < t.cnt) ? p[i] : 0.f;
}

template <int V, int MODE>
__device__ __forceinline__ void load_bf16(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const uint16_t* p = (const uint16_t*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (t.vec) {
      const uint4 w = *(const uint4*)p;
      d[0] = bf16_lo(w.x); d[1] = bf16_hi(w.x); d[2] = bf16_lo(w.y); d[3] = bf16_hi(w.y);
      d[4] = bf16_lo(w.z); d[5] = bf16_hi(w.z); d[6] = bf16_lo(w.w); d[7] = bf16_hi(w.w);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = (i < t.cnt) ? bf16_at(p + i) : 0.f;
}

template <int V, int MODE>
__device__ __forceinline__ void load_u8(float (&d)[V], const ExecArgs& a, int slot, const Tile& t) {
  const uint8_t* p = (const uint8_t*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (t.vec) {
      const uint2 w = *(const uint2*)p;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = (float)((w.x >> (8 * i)) & 0xFFu);
#pragma unroll
      for (int i = 0; i < 4; ++i) d[4 + i] = (float)((w.y >> (8 * i)) & 0xFFu);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = (i < t.cnt) ? (float)p[i] : 0.f;
}

template <int V, int MODE>
__device__ __forceinline__ void store_f32(const float (&s)[V], const ExecArgs& a, int slot, const Tile& t) {
  float* p = (float*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (t.vec) {
      *(float4*)p = make_float4(s[0], s[1], s[2], s[3]);
      *(float4*)(p + 4) = make_float4(s[4], s[5], s[6], s[7]);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (i < t.cnt) p[i] = s[i];
}

template <int V, int MODE>
__device__ __forceinline__ void store_bf16(const float (&s)[V], const ExecArgs& a, int slot, const Tile& t) {
  uint16_t* p = (uint16_t*)a.ptr[slot] + elem_offset<V, MODE>(a, slot, t);
  if (MODE == M_ELEM && V == 8) {
    if (t.vec) {
      *(uint4*)p = make_uint4(pack_bf16(s[0], s[1]), pack_bf16(s[2], s[3]),
                              pack_bf16(s[4], s[5]), pack_bf16(s[6], s[7]));
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (i < t.cnt) p[i] = (uint16_t)(pack_bf16(s[i], 0.f) & 0xFFFFu);
}

// ---------------------------------------------------------------- ops
template <int V, int F>
__device__ __forceinline__ void unary(float (&r)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const float x = r[i];
    float y;
    if (F == F_EXP) y = expf(x);
    else if (F == F_TANH) y = tanhf(x);
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

template <int V, int F>
__device__ __forceinline__ void binary(float (&l)[V], const float (&r)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (F == F_ADD) l[i] = l[i] + r[i];
    else if (F == F_SUB) l[i] = l[i] - r[i];
    else if (F == F_MUL) l[i] = l[i] * r[i];
    else if (F == F_DIV) l[i] = l[i] / r[i];
    else if (F == F_MAX) l[i] = fmaxf(l[i], r[i]);
    else l[i] = fminf(l[i], r[i]);  // F_MIN
  }
}

template <int V, int OP>
__device__ __forceinline__ void xvec(float (&r)[V], const float* x) {  // x: V values
  if (V == 8) {
    const float4 a = *(const float4*)x;
    const float4 b = *(const float4*)(x + 4);
    const float xs[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < V; ++i) r[i] = xop<OP>(r[i], xs[i % 8]);
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

template <int V>
__device__ __forceinline__ void copy(float (&d)[V], const float (&s)[V]) {
#pragma unroll
  for (int i = 0; i < V; ++i) d[i] = s[i];
}

template <int V, int D>
__device__ __forceinline__ void pick(float (&R)[kNR][V], int src) {
  switch (src) {
    case 0: copy<V>(R[D], R[0]); break;
    case 1: copy<V>(R[D], R[1]); break;
    case 2: copy<V>(R[D], R[2]); break;
    case 3: copy<V>(R[D], R[3]); break;
    case 4: copy<V>(R[D], R[4]); break;
    case 5: copy<V>(R[D], R[5]); break;
    case 6: copy<V>(R[D], R[6]); break;
    default: copy<V>(R[D], R[7]); break;
  }
}

// ---------------------------------------------------------------- interpreter
template <int V, int MODE>
__device__ __forceinline__ void interpret(const ExecArgs& a, const Instr* prog, int n,
                                          const Tile& t, float* lds_col, float* lds_row,
                                          float& acc, bool store_global) {
  float R[kNR][V];
#pragma unroll
  for (int s = 0; s < kNR; ++s)
#pragma unroll
    for (int i = 0; i < V; ++i) R[s][i] = 0.f;

  for (int pc = 0; pc < n; ++pc) {
    const Instr ins = prog[pc];
    const int arg = ins.arg;
    switch (ins.code) {
#define GTF_SLOT_CASES(D)                                                                  \
  case F_LD_F32 * kNR + D: load_f32<V, MODE>(R[D], a, arg, t); break;                    \
  case F_LD_BF16 * kNR + D: load_bf16<V, MODE>(R[D], a, arg, t); break;                  \
  case F_LD_U8 * kNR + D: load_u8<V, MODE>(R[D], a, arg, t); break;                      \
  case F_PUSH_IMM * kNR + D:                                                               \
    for (int i = 0; i < V; ++i) R[D][i] = ins.imm;                                         \
    break;                                                                                 \
  case F_PICK * kNR + D: pick<V, D>(R, arg); break;                                      \
  case F_EXP * kNR + D: unary<V, F_EXP>(R[D]); break;                                    \
  case F_TANH * kNR + D: unary<V, F_TANH>(R[D]); break;                                  \
  case F_SIGMOID * kNR + D: unary<V, F_SIGMOID>(R[D]); break;                            \
  case F_RELU * kNR + D: unary<V, F_RELU>(R[D]); break;                                  \
  case F_GELU * kNR + D: unary<V, F_GELU>(R[D]); break;                                  \
  case F_SQUARE * kNR + D: unary<V, F_SQUARE>(R[D]); break;                              \
  case F_SQRT * kNR + D: unary<V, F_SQRT>(R[D]); break;                                  \
  case F_RECIP * kNR + D: unary<V, F_RECIP>(R[D]); break;                                \
  case F_NEG * kNR + D: unary<V, F_NEG>(R[D]); break;                                    \
  case F_ADD * kNR + D: binary<V, F_ADD>(R[D], R[(D + 1) % kNR]); break;                 \
  case F_SUB * kNR + D: binary<V, F_SUB>(R[D], R[(D + 1) % kNR]); break;                 \
  case F_MUL * kNR + D: binary<V, F_MUL>(R[D], R[(D + 1) % kNR]); break;                 \
  case F_DIV * kNR + D: binary<V, F_DIV>(R[D], R[(D + 1) % kNR]); break;                 \
  case F_MAX * kNR + D: binary<V, F_MAX>(R[D], R[(D + 1) % kNR]); break;                 \
  case F_MIN * kNR + D: binary<V, F_MIN>(R[D], R[(D + 1) % kNR]); break;                 \
  case (F_ADD_I + X_ADD) * kNR + D: xscalar<V, X_ADD>(R[D], ins.imm); break;             \
  case (F_ADD_I + X_SUB) * kNR + D: xscalar<V, X_SUB>(R[D], ins.imm); break;             \
  case (F_ADD_I + X_RSUB) * kNR + D: xscalar<V, X_RSUB>(R[D], ins.imm); break;           \
  case (F_ADD_I + X_MUL) * kNR + D: xscalar<V, X_MUL>(R[D], ins.imm); break;             \
  case (F_ADD_I + X_DIV) * kNR + D: xscalar<V, X_DIV>(R[D], ins.imm); break;             \
  case (F_ADD_I + X_RDIV) * kNR + D: xscalar<V, X_RDIV>(R[D], ins.imm); break;           \
  case (F_ADD_I + X_MAX) * kNR + D: xscalar<V, X_MAX>(R[D], ins.imm); break;             \
  case (F_ADD_I + X_MIN) * kNR + D: xscalar<V, X_MIN>(R[D], ins.imm); break;             \
  case F_ST_F32 * kNR + D:                                                                 \
    if (MODE == M_ELEM || store_global) store_f32<V, MODE>(R[D], a, arg, t);              \
    break;                                                                                 \
  case F_ST_BF16 * kNR + D:                                                                \
    if (MODE == M_ELEM || store_global) store_bf16<V, MODE>(R[D], a, arg, t);             \
    break;                                                                                 \
  case F_RED * kNR + D:                                                                    \
    if (MODE == M_ELEM) {                                                                  \
      for (int i = 0; i < V; ++i)                                                          \
        if (t.vec || i < t.cnt) acc += R[D][i];                                            \
    }                                                                                      \
    break;                                                                                 \
  case F_ST_LDS * kNR + D:                                                                 \
    if (MODE == M_ROW) lds_row[arg * a.RB + t.rr] = R[D][0];                               \
    if (MODE == M_COL) lds_col[arg * a.PW + t.cl] = R[D][0];                               \
    break;                                                                                 \
  case F_PUSH_COL * kNR + D:                                                               \
    if (MODE == M_ELEM) {                                                                  \
      for (int i = 0; i < V; ++i) R[D][i] = lds_col[arg * a.PW + t.cl + i];               \
    }                                                                                      \
    break;                                                                                 \
  case F_PUSH_ROW * kNR + D:                                                               \
    if (MODE == M_ELEM) {                                                                  \
      const float x = lds_row[arg * a.RB + t.rr];                                          \
      for (int i = 0; i < V; ++i) R[D][i] = x;                                             \
    }                                                                                      \
    break;                                                                                 \
  case (F_ADD_C + X_ADD) * kNR + D:                                                        \
    if (MODE == M_ELEM) xvec<V, X_ADD>(R[D], lds_col + arg * a.PW + t.cl);                \
    break;                                                                                 \
  case (F_ADD_C + X_SUB) * kNR + D:                                                        \
    if (MODE == M_ELEM) xvec<V, X_SUB>(R[D], lds_col + arg * a.PW + t.cl);                \
    break;                                                                                 \
  case (F_ADD_C + X_RSUB) * kNR + D:                                                       \
    if (MODE == M_ELEM) xvec<V, X_RSUB>(R[D], lds_col + arg * a.PW + t.cl);               \
    break;                                                                                 \
  case (F_ADD_C + X_MUL) * kNR + D:                                                        \
    if (MODE == M_ELEM) xvec<V, X_MUL>(R[D], lds_col + arg * a.PW + t.cl);                \
    break;                                                                                 \
  case (F_ADD_C + X_DIV) * kNR + D:                                                        \
    if (MODE == M_ELEM) xvec<V, X_DIV>(R[D], lds_col + arg * a.PW + t.cl);                \
    break;                                                                                 \
  case (F_ADD_C + X_RDIV) * kNR + D:                                                       \
    if (MODE == M_ELEM) xvec<V, X_RDIV>(R[D], lds_col + arg * a.PW + t.cl);               \
    break;                                                                                 \
  case (F_ADD_C + X_MAX) * kNR + D:                                                        \
    if (MODE == M_ELEM) xvec<V, X_MAX>(R[D], lds_col + arg * a.PW + t.cl);                \
    break;                                                                                 \
  case (F_ADD_C + X_MIN) * kNR + D:                                                        \
    if (MODE == M_ELEM) xvec<V, X_MIN>(R[D], lds_col + arg * a.PW + t.cl);                \
    break;                                                                                 \
  case (F_ADD_R + X_ADD) * kNR + D:                                                        \
    if (MODE == M_ELEM) xscalar<V, X_ADD>(R[D], lds_row[arg * a.RB + t.rr]);              \
    break;                                                                                 \
  case (F_ADD_R + X_SUB) * kNR + D:                                                        \
    if (MODE == M_ELEM) xscalar<V, X_SUB>(R[D], lds_row[arg * a.RB + t.rr]);              \
    break;                                                                                 \
  case (F_ADD_R + X_RSUB) * kNR + D:                                                       \
    if (MODE == M_ELEM) xscalar<V, X_RSUB>(R[D], lds_row[arg * a.RB + t.rr]);             \
    break;                                                                                 \
  case (F_ADD_R + X_MUL) * kNR + D:                                                        \
    if (MODE == M_ELEM) xscalar<V, X_MUL>(R[D], lds_row[arg * a.RB + t.rr]);              \
    break;                                                                                 \
  case (F_ADD_R + X_DIV) * kNR + D:                                                        \
    if (MODE == M_ELEM) xscalar<V, X_DIV>(R[D], lds_row[arg * a.RB + t.rr]);              \
    break;                                                                                 \
  case (F_ADD_R + X_RDIV) * kNR + D:                                                       \
    if (MODE == M_ELEM) xscalar<V, X_RDIV>(R[D], lds_row[arg * a.RB + t.rr]);             \
    break;                                                                                 \
  case (F_ADD_R + X_MAX) * kNR + D:                                                        \
    if (MODE == M_ELEM) xscalar<V, X_MAX>(R[D], lds_row[arg * a.RB + t.rr]);              \
    break;                                                                                 \
  case (F_ADD_R + X_MIN) * kNR + D:                                                        \
    if (MODE == M_ELEM) xscalar<V, X_MIN>(R[D], lds_row[arg * a.RB + t.rr]);              \
    break;

      GTF_SLOT_CASES(0)
      GTF_SLOT_CASES(1)
      GTF_SLOT_CASES(2)
      GTF_SLOT_CASES(3)
      GTF_SLOT_CASES(4)
      GTF_SLOT_CASES(5)
      GTF_SLOT_CASES(6)
      GTF_SLOT_CASES(7)
#undef GTF_SLOT_CASES
      default:
        break;
    }
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

__device__ __forceinline__ void store_reduced(const ExecArgs& a, int64_t row, float s) {
  const float v = a.reduce == 2 ? s / (float)a.C : s;
  const int slot = a.red_slot;
  const int64_t off = row * a.rstride[slot];
  if (a.red_dtype == DT_BF16)
    ((uint16_t*)a.ptr[slot])[off] = (uint16_t)(pack_bf16(v, 0.f) & 0xFFFFu);
  else
    ((float*)a.ptr[slot])[off] = v;
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
        interpret<1, M_COL>(a, col_prog, a.n_col, t, lds_col, lds_row, dummy, rb == 0);
      }
      __syncthreads();
      staged = true;
    }
    if (a.n_row > 0) {
      __syncthreads();
      for (int r = tid; r < nr; r += kBlock) {
        Tile t{r0 + r, 0, 0, 0, r, 1, false};
        interpret<1, M_ROW>(a, row_prog, a.n_row, t, lds_col, lds_row, dummy, p == 0);
      }
      __syncthreads();
    }

    const int npass = (nr + rpp - 1) / rpp;
    for (int pass = 0; pass < npass; ++pass) {
      const int rr = pass * rpp + sub;
      float acc = 0.f;
      if (rr < nr && a.n_elem > 0) {
        const int64_t row = r0 + rr;
        for (int cl = lt * kV; cl < nc; cl += tpr * kV) {
          Tile t;
          t.row = row;
          t.col = c0 + cl;
          t.eoff = row * erow_stride + t.col;
          t.cl = cl;
          t.rr = rr;
          t.cnt = min(kV, nc - cl);
          t.vec = a.vec_ok && t.cnt == kV;
          interpret<kV, M_ELEM>(a, el_prog, a.n_elem, t, lds_col, lds_row, acc, true);
        }
      }
      if (a.reduce) {
        const int w = min(tpr, 64);
        float s = segment_sum(acc, w);
        if (tpr <= 64) {
          if (lt == 0 && rr < nr) store_reduced(a, r0 + rr, s);
        } else {
          // rows wider than a wave: combine the per-wave sums through LDS
          const int wpr = tpr >> 6;        // waves per row
          if ((tid & 63) == 0) lds_red[tid >> 6] = s;
          __syncthreads();
          if (lt == 0 && rr < nr) {
            float tot = 0.f;
            for (int k = 0; k < wpr; ++k) tot += lds_red[sub * wpr + k];
            store_reduced(a, r0 + rr, tot);
          }
          __syncthreads();
        }
      }
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
