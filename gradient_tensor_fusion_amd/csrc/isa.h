// isa.h -- the op-program format shared by the host group compiler and the
// executor kernel.
//
// A fused group (TVM "Operator Fusion": FuseOps groups, FuseTIR merges the
// group's functions so intermediates never reach device memory) runs as one
// launch of an interpreter over a small stack machine whose slots are
// vector registers.  The host compiles each group into up to three
// programs:
//
//   column phase  once per column of the staged panel (values shaped [1,C]);
//                 results go to LDS column slots.
//   row phase     once per row of the row block (values shaped [R,1]);
//                 results go to LDS row slots.
//   element phase once per tile of kV consecutive elements of one row;
//                 reads rows/columns from LDS, streams [R,C] tensors.
//
// Each instruction is {code, arg, imm}.  code = form * kNR + d, where d is
// the slot the instruction writes (or reads, for stores and reductions), so
// every register access in the kernel has a compile-time index and the
// slots stay in VGPRs.  Dispatch is wave-uniform (the program is the same
// for every lane), a scalar branch per instruction.
#pragma once

#include <stdint.h>

namespace gtf {

constexpr int kV = 8;            // elements per lane per tile
constexpr int kNR = 8;           // stack slots
constexpr int kMaxInstr = 288;   // instructions over all three phases
constexpr int kMaxSlots = 16;    // external tensors of one group
constexpr int kMaxLdsCol = 4;    // LDS column slots
constexpr int kMaxLdsRow = 8;    // LDS row slots
constexpr int kBlock = 256;      // threads per workgroup
constexpr int kPanelMax = 4096;  // widest column panel staged in LDS

enum Form : int {
  // push from memory: arg = external tensor slot
  F_LD_F32 = 0, F_LD_BF16, F_LD_U8,
  // push a broadcast value: arg = LDS column slot / LDS row slot; imm
  F_PUSH_COL, F_PUSH_ROW, F_PUSH_IMM,
  // push a copy of slot arg
  F_PICK,
  // unary, in place on slot d
  F_EXP, F_TANH, F_SIGMOID, F_RELU, F_GELU, F_SQUARE, F_SQRT, F_RECIP, F_NEG,
  // binary on slots d (left) and d+1 (right), result in d
  F_ADD, F_SUB, F_MUL, F_DIV, F_MAX, F_MIN,
  // slot d = slot d (op) X, X = LDS column slot arg
  F_ADD_C, F_SUB_C, F_RSUB_C, F_MUL_C, F_DIV_C, F_RDIV_C, F_MAX_C, F_MIN_C,
  // X = LDS row slot arg
  F_ADD_R, F_SUB_R, F_RSUB_R, F_MUL_R, F_DIV_R, F_RDIV_R, F_MAX_R, F_MIN_R,
  // X = imm
  F_ADD_I, F_SUB_I, F_RSUB_I, F_MUL_I, F_DIV_I, F_RDIV_I, F_MAX_I, F_MIN_I,
  // store slot d to external tensor slot arg (no pop)
  F_ST_F32, F_ST_BF16,
  // add slot d into the row accumulator (element phase only)
  F_RED,
  // store slot d to LDS slot arg (column slot in the column phase, row slot
  // in the row phase)
  F_ST_LDS,
  F_COUNT
};

// binary-with-X forms are laid out as 8 consecutive ops per operand class
enum XOp : int { X_ADD = 0, X_SUB, X_RSUB, X_MUL, X_DIV, X_RDIV, X_MAX, X_MIN };

struct Instr {
  uint16_t code;  // form * kNR + d
  uint16_t arg;
  float imm;
};

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_U8 = 2 };

// Kernel arguments, passed by value (kernarg segment; read with scalar
// loads).  Strides are in elements.
struct ExecArgs {
  int64_t R, C;            // domain
  int64_t n_items;         // row blocks x panels
  int32_t n_panels, RB, PW;    // panels, rows per block, panel width
  int32_t tpr_log2;        // threads per row = 1 << tpr_log2 (<= kBlock)
  int32_t n_col, n_row, n_elem;  // program lengths (programs back to back)
  int32_t n_col_slots, n_row_slots;
  int32_t reduce;          // 0 none, 1 sum, 2 mean
  int32_t red_dtype;       // reduce output dtype
  int32_t red_slot;        // external slot of the reduce output
  int32_t vec_ok;          // element tensors and rows are 16-byte aligned
  int32_t pad0;
  void* ptr[kMaxSlots];
  int64_t rstride[kMaxSlots];
  int64_t cstride[kMaxSlots];
  Instr prog[kMaxInstr];
};

// Bucket chunk: a run of at most kChunkElems elements of one tensor.
constexpr int kChunkElems = 16384;
constexpr int kMaxBucketPtrs = 256;  // tensor + bucket pointers per launch

struct Chunk {
  int64_t t_off;      // element offset inside the tensor
  int64_t b_off;      // element offset inside the bucket
  int32_t n;          // elements
  uint16_t t_slot;    // pointer slot of the tensor (local to the launch)
  uint16_t b_slot;    // pointer slot of the bucket (local to the launch)
};

struct BucketArgs {
  const Chunk* chunks;   // this launch's chunks (device memory)
  float scale;
  int32_t unpack;        // 0: tensor -> bucket, 1: bucket -> tensor
  int32_t dtype;         // DT_F32 / DT_BF16
  int32_t n_chunks;
  void* ptr[kMaxBucketPtrs];
};

}  // namespace gtf
