// isa.h -- the op-program format shared by the host group compiler and the
// executor kernel.
//
// A fused group (TVM "Operator Fusion": FuseOps groups, FuseTIR merges the
// group's functions so intermediates never reach device memory) runs as one
// launch of an interpreter whose values are vector registers.  The host
// compiles each group into up to three programs:
//
//   column phase  once per column of the staged panel (values shaped [1,C]);
//                 results go to LDS column slots.
//   row phase     once per row of the row block (values shaped [R,1]);
//                 results go to LDS row slots.  A group may hold up to
//                 kMaxStages element stages, each ending in a row
//                 reduction whose result later stages read (row-resident
//                 reduce-then-broadcast, e.g. a one-kernel LayerNorm); a
//                 row program runs before each stage.
//   element phase once per tile of one row; reads rows/columns from LDS,
//                 streams [R,C] tensors.  A lane's tile is K sub-tiles of
//                 kV consecutive elements, tpr * kV elements apart in the
//                 row, so one dispatched instruction covers K * kV
//                 elements per lane (K = 4 in the wide instance).
//
// The machine has two working registers A and B and NS spill slots, each
// holding one tile.  Every op writes A, reading A (and B), or B alone for
// the unary and immediate forms that keep an operand needed later in B;
// moves between A, B and the slots are explicit instructions.  Each instruction form has
// exactly one body in the kernel, and every register index is a
// compile-time constant, so the registers stay in VGPRs.  Three kernel
// instances exist: wide with no spill slot (K = 4, NS = 0: A and B only,
// the highest occupancy), wide with two (K = 4, NS = 2: 4 x 32 VGPRs of
// registers), and narrow (K = 1, NS = 6) for programs that need more.
#pragma once

#include <stdint.h>

namespace gtf {

constexpr int kV = 8;            // elements per lane per sub-tile (one 16-byte bf16 load)
constexpr int kNS = 6;           // spill slots of the narrow instance
constexpr int kWideK = 4;        // sub-tiles per lane tile in the wide instance
constexpr int kWideNS = 2;       // spill slots of the wide instance
constexpr int kMaxInstr = 320;   // instructions over all three phases
constexpr int kMaxSlots = 16;    // external tensors of one group
constexpr int kMaxLdsCol = 4;    // LDS column slots
constexpr int kMaxLdsRow = 8;    // LDS row slots
constexpr int kBlock = 256;      // threads per workgroup
constexpr int kPanelMax = 4096;  // widest column panel staged in LDS
constexpr int kMaxStages = 4;    // element stages of one group (row-resident reductions)

enum Form : int {
  // load a tile of external tensor slot `arg` into A / into B
  F_LD_F32_A = 0, F_LD_BF16_A, F_LD_U8_A, F_LD_F32_B, F_LD_BF16_B, F_LD_U8_B,
  // broadcast value into A / B: LDS column slot arg, LDS row slot arg, imm
  F_COL_A, F_ROW_A, F_IMM_A, F_COL_B, F_ROW_B, F_IMM_B,
  // moves
  F_A2B, F_B2A,
  F_A2S0, F_A2S1, F_A2S2, F_A2S3, F_A2S4, F_A2S5,
  F_B2S0, F_B2S1, F_B2S2, F_B2S3, F_B2S4, F_B2S5,
  F_S02A, F_S12A, F_S22A, F_S32A, F_S42A, F_S52A,
  F_S02B, F_S12B, F_S22B, F_S32B, F_S42B, F_S52B,
  // A = f(A)
  F_EXP, F_TANH, F_SIGMOID, F_RELU, F_GELU, F_SQUARE, F_SQRT, F_RECIP, F_NEG,
  // A = A op B (RSUB: B - A, RDIV: B / A)
  F_ADD, F_SUB, F_RSUB, F_MUL, F_DIV, F_RDIV, F_MAX, F_MIN,
  // A = A op X, X = LDS column slot arg / LDS row slot arg / imm
  F_ADD_C, F_SUB_C, F_RSUB_C, F_MUL_C, F_DIV_C, F_RDIV_C, F_MAX_C, F_MIN_C,
  F_ADD_R, F_SUB_R, F_RSUB_R, F_MUL_R, F_DIV_R, F_RDIV_R, F_MAX_R, F_MIN_R,
  F_ADD_I, F_SUB_I, F_RSUB_I, F_MUL_I, F_DIV_I, F_RDIV_I, F_MAX_I, F_MIN_I,
  // store A to external tensor slot arg
  F_ST_F32, F_ST_BF16,
  // add A into the row accumulator (element phase)
  F_RED,
  // store A to LDS slot arg (column slot in the column phase, row slot in
  // the row phase)
  F_ST_LDS,
  // addressed loads into A (element phase): element (row, col) of slot arg
  // at row * rstride + col * cstride, element by element (a transpose)
  F_LDG_F32_A, F_LDG_BF16_A,
  // concat along columns (element or column phase): slots arg & 0xFF and
  // arg >> 8, split at column imm; each side at its own strides
  F_LDC_F32_A, F_LDC_BF16_A,
  // the item's transposed tile staged in LDS, into A (element phase)
  F_LDT_A,
  // A = gelu(A) to about 1e-5 relative, for a result that is rounded to
  // bf16 and read by nothing else
  F_GELU_BF,
  // fold A into the row accumulator with max (element phase)
  F_RED_MAX,
  // fold A into a paired accumulator (element phase): (mean, squared
  // deviations, count), or (max, sum of exp(x - max))
  F_RED_MV, F_RED_SE,
  // A = f(B), B unchanged, for the short unary forms (each form's body is
  // one more copy of its code in every kernel instance)
  F_EXP_B, F_TANH_B, F_RELU_B, F_SQUARE_B, F_NEG_B,
  // A = B op imm, B unchanged (the order of the XOp family)
  F_ADD_IB, F_SUB_IB, F_RSUB_IB, F_MUL_IB, F_DIV_IB, F_RDIV_IB, F_MAX_IB, F_MIN_IB,
  F_COUNT
};

// binary ops in the order of the A op B / A op X families
enum XOp : int { X_ADD = 0, X_SUB, X_RSUB, X_MUL, X_DIV, X_RDIV, X_MAX, X_MIN };

struct Instr {
  uint16_t code;  // Form
  uint16_t arg;
  float imm;
};

enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_U8 = 2 };

// One work item of a multi-set run: elements [off, off + n) (n <= the
// panel width) of every tensor of set `set`.
struct MultiItem {
  int64_t off;
  int32_t n;
  int32_t set;
};

// One element stage: the row program that runs before it, its element
// program, and the row reduction it ends in (if any), whose per-row result
// goes to an LDS row slot (read by later stages and row programs) and/or
// to an external slot.  A group without row-resident reductions has one
// stage.
struct StageDesc {
  int32_t row_off, row_len;  // row program (instruction offset, length)
  int32_t el_off, el_len;    // element program
  int32_t red;               // 0 none, 1 row sum, 2 row mean, 3 row max,
                             // paired (two results in one pass): 4 mean and
                             // mean of squared deviations from it, 5 max and
                             // sum of exp(x - max)
  int32_t red_lds;           // LDS row slot for the result, or -1
  int32_t red_slot;          // external slot for the result, or -1
  int32_t red_dtype;         // its dtype
  int32_t red2_lds, red2_slot, red2_dtype;  // the second result of a paired one
  int32_t red2_pad_;
};

// Kernel arguments, passed by value (kernarg segment; read with scalar
// loads).  Strides are in elements.
struct ExecArgs {
  int64_t R, C;            // domain
  int64_t n_items;         // row blocks x panels
  int32_t n_panels, RB, PW;    // panels, rows per block, panel width
  int32_t tpr_log2;        // threads per row = 1 << tpr_log2 (<= kBlock)
  int32_t n_col;           // column program length (at offset 0)
  int32_t n_stages;        // element stages (>= 1)
  StageDesc stage[kMaxStages];
  int32_t n_col_slots, n_row_slots;
  uint32_t vec_slots;      // bit s: slot s takes 16-byte (u8: 8-byte) accesses
  int32_t K;               // sub-tiles per lane tile: kWideK (wide) or 1 (narrow)
  int32_t NS;              // spill slots of the instance: 0, kWideNS or kNS
  // multi-set run of a flat group (null otherwise): item table, one row of
  // n_slots pointers per set and one 16-byte-access mask per set
  const MultiItem* m_items;
  void* const* m_ptrs;
  const uint32_t* m_vec;
  int32_t n_slots;
  int32_t slow_only;       // 1: every tile goes sub-tile by sub-tile (addressed loads)
  // a transposed source staged per item in LDS (n_tr = 0 or 1): slot
  // tr_slot holds X, the item's tile is X rows c0.. (domain columns) by
  // elements r0.. (domain rows); tile row stride tr_stride > PW floats
  // (every column a lane of a run may read, plus one)
  int32_t n_tr, tr_slot, tr_bf16, tr_stride;
  int32_t tr_off;          // the tile's offset in LDS, in floats
  int32_t tr_vec;          // 1: the source allows 16-byte reads along its rows
  int32_t tr_pad_;
  void* ptr[kMaxSlots];
  int64_t rstride[kMaxSlots];
  int64_t cstride[kMaxSlots];
  Instr prog[kMaxInstr];
};

static_assert(sizeof(ExecArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// Bucket chunk: a run of one tensor of at most kChunkBytes bytes (4096 fp32
// or 8192 bf16 elements), what one workgroup of the bucket kernel moves
// with all of its loads in flight together.
constexpr int kChunkBytes = 16384;
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
