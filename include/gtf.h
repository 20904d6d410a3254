/*
 * gtf.h -- fused operator groups and tensor-fusion buckets on one AMD
 * Instinct MI355X (gfx950).  Plain C ABI: every function is extern "C",
 * takes plain pointers and sizes, returns an int status (0 = GTF_OK,
 * negative = error) and never throws.  After a negative status,
 * gtf_last_error() returns a message for the calling thread.
 *
 * Two parts:
 *
 * 1. Fused operator groups.  A program (tensors + ops in topological order)
 *    is annotated with TVM's OpPatternKind, its post-dominator tree is
 *    built, and ops are grouped by the post-dominator fusion rules (Apache
 *    TVM, "Operator Fusion": sections "Operator Pattern Classification",
 *    "FuseOps: Automatic Fusion" / "Algorithm" and "Fusion rules").  Each
 *    group then becomes one function over its external tensors (same page,
 *    "Example" and "FuseTIR"): here, one launch of a register-resident
 *    op-program kernel whose intermediates never touch device memory (DisCo,
 *    arXiv 2209.12769, section 1: op fusion keeps intermediate results out of
 *    device memory and saves launches).
 *
 * 2. Tensor-fusion buckets.  Many small gradient tensors are packed into
 *    contiguous buckets whose size is the sum of the member sizes, under a
 *    size threshold, scaled by 1/N for the data-parallel average, and
 *    unpacked back (DisCo section 1 "tensor fusion" and "AllReduce ... sums
 *    (or averages)"; section 7, Horovod's fusion threshold).  One launch
 *    covers hundreds of tensors through a device-side chunk table.
 *
 * Memory ownership: the caller owns every device buffer (inputs, outputs,
 * stored intermediates, bucket buffers, the bucket workspace).  The library
 * owns only its host-side plan objects.  It never allocates device memory
 * and never synchronises a stream.  All run calls are asynchronous on the
 * HIP stream passed in (a hipStream_t cast to void*; NULL is the null
 * stream).
 *
 * Tensors are dense, row-major, at most rank 2.  A rank-1 tensor [N] is
 * treated as the row vector [1, N].  Binary and ternary ops broadcast
 * NumPy-style: each operand is [R,C], [1,C], [R,1] or [1,1] against the
 * result [R,C].  Arithmetic is fp32 (bf16 and u8 inputs widen exactly);
 * a bf16 store rounds to nearest-even once.
 */
#ifndef GTF_H
#define GTF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GTF_ABI_VERSION 2u

/* ---- status codes ---------------------------------------------------- */
enum {
  GTF_OK = 0,
  GTF_E_INVALID = -1,     /* NULL argument, bad index, order/cycle, bad version */
  GTF_E_UNSUPPORTED = -2, /* opcode, dtype or rank this library does not run */
  GTF_E_SHAPE = -3,       /* shapes that do not broadcast or do not match */
  GTF_E_LIMIT = -4,       /* a per-group or per-plan resource limit */
  GTF_E_STATE = -5,       /* call out of order (bucket run before bind) */
  GTF_E_HIP = -6          /* a HIP runtime call or launch failed */
};

/* ---- element types, tensor roles ------------------------------------- */
enum { GTF_F32 = 0, GTF_BF16 = 1, GTF_U8 = 2 };
enum { GTF_ROLE_IN = 0, GTF_ROLE_OUT = 1, GTF_ROLE_TMP = 2 };

/* ---- OpPatternKind (values as in TVM's table) ------------------------ */
enum {
  GTF_PAT_ELEMWISE = 0,
  GTF_PAT_BROADCAST = 1,
  GTF_PAT_INJECTIVE = 2,
  GTF_PAT_COMM_REDUCE = 3,
  GTF_PAT_OUT_EWISE_FUSABLE = 4,
  GTF_PAT_TUPLE = 7,
  GTF_PAT_OPAQUE = 8
};

/* ---- opcodes ---------------------------------------------------------
 * unary (n_in 1):  copy (injective; same shape), exp, tanh,
 *                  sigmoid = 1/(1+exp(-x)), relu = x>0 ? x : +0,
 *                  gelu = x/2*erfc(-x/sqrt 2), square = x*x, sqrt,
 *                  recip = 1/x, neg
 * immediate:       add_imm = x + imm, mul_imm = x * imm
 * binary (n_in 2): add, sub, mul, div (a op b), max, min
 * ternary:         add3 = (a + b) + c
 * dropout:         dmul (n_in 2: h, mask) = (h * imm) * mask
 * row reduce:      row_sum, row_mean, row_max over the last axis; the
 *                  output is declared [R, 1]; the mean divides the sum by
 *                  the width; the max is exact (any order gives it), and
 *                  of an empty row (C = 0) it is -inf.  All three are
 *                  kCommReduce (TVM "Operator Pattern Classification").
 * injective data movement (kInjective, TVM "Operator Pattern
 * Classification": each output element is one input element, moved):
 *                  transpose: [R, C] (rank 2) -> [C, R];
 *                  reshape: any shape -> the declared shape of the same
 *                  element count, row-major order kept;
 *                  concat (n_in 2): [R, C1] ++ [R, C2] -> [R, C1 + C2]
 *                  along the last axis (rank 2, C1, C2 >= 1, one dtype);
 *                  concat (n_in 1) of a tuple: its fields along the last
 *                  axis.
 *                  Inside a group these run as addressed loads: their
 *                  inputs come from memory, or, for a concat or a tuple,
 *                  from a transpose or reshape of a tensor in memory that
 *                  nothing else reads and that keeps its dtype (folded
 *                  into the load's addressing).
 * tuple (kTuple, TVM "Operator Pattern Classification"; n_in 2): the
 *                  fields [R, C1], [R, C2] (rank 2, one dtype), declared
 *                  [R, C1 + C2]: a tuple's value is its fields side by
 *                  side, so a concat of it is that value.  Read only by
 *                  concats (n_in 1) and never a graph output.  A tuple
 *                  fuses into the concat that reads it in phase 1, and
 *                  producers of its fields no more complex than injective
 *                  join that group in phase 2 (TVM "Fusion rules").
 * add/sub/mul/div/max/min/add3/dmul broadcast their operands; sqrt and
 * div are correctly rounded; no multiply-add is ever contracted. */
enum {
  GTF_OP_COPY = 0, GTF_OP_EXP = 1, GTF_OP_TANH = 2, GTF_OP_SIGMOID = 3,
  GTF_OP_RELU = 4, GTF_OP_GELU = 5, GTF_OP_SQUARE = 6, GTF_OP_SQRT = 7,
  GTF_OP_RECIP = 8, GTF_OP_NEG = 9,
  GTF_OP_ADD_IMM = 16, GTF_OP_MUL_IMM = 17,
  GTF_OP_ADD = 32, GTF_OP_SUB = 33, GTF_OP_MUL = 34, GTF_OP_DIV = 35,
  GTF_OP_MAX = 36, GTF_OP_MIN = 37,
  GTF_OP_ADD3 = 48, GTF_OP_DMUL = 49,
  GTF_OP_ROW_SUM = 64, GTF_OP_ROW_MEAN = 65, GTF_OP_ROW_MAX = 66,
  GTF_OP_TRANSPOSE = 80, GTF_OP_RESHAPE = 81, GTF_OP_CONCAT = 82, GTF_OP_TUPLE = 83
};

#define GTF_OPF_OPAQUE 1 /* op flag: force OpPatternKind kOpaque (a barrier) */

typedef struct {
  int32_t dtype;    /* GTF_F32 / GTF_BF16 / GTF_U8 (u8 only as an input)   */
  int32_t rank;     /* 1 or 2                                              */
  int64_t shape[2]; /* shape[0..rank-1], each >= 0                         */
  int32_t role;     /* GTF_ROLE_*                                          */
  int32_t reserved; /* must be 0                                           */
} gtf_tensor_desc;

typedef struct {
  int32_t opcode; /* GTF_OP_*                                              */
  int32_t n_in;   /* number of inputs, as the opcode requires             */
  int32_t in[3];  /* input tensor ids (index into the tensor array)       */
  int32_t out;    /* output tensor id                                     */
  float imm;      /* immediate for add_imm / mul_imm / dmul               */
  int32_t flags;  /* GTF_OPF_*                                            */
} gtf_op_desc;

typedef struct {
  uint32_t abi_version; /* GTF_ABI_VERSION                                */
  int32_t n_tensors;
  const gtf_tensor_desc* tensors;
  int32_t n_ops;
  const gtf_op_desc* ops; /* topological: an op reads only inputs and
                             outputs of earlier ops                       */
} gtf_program_desc;

/* ---- limits ------------------------------------------------------------
 * kMaxFusedOps is 256 on the TVM page; the page names a maximum argument
 * count without its value, here 16 external tensors per group.  A fusion
 * whose compiled op-program would not fit the kernel's register stack or
 * instruction buffer is refused like one over the argument limit. */
#define GTF_MAX_GROUP_OPS 256
#define GTF_MAX_GROUP_ARGS 16

/* fuse_plan_create flags */
#define GTF_NO_FUSE 1u /* one op per group: the unfused baseline            */
/* Row-resident extension of the fusion rules: after TVM's three phases, a
 * group ending in a row reduction is merged with a group on the same [R,C]
 * domain that reads the reduction's result (reduce-then-broadcast, e.g. a
 * LayerNorm in one kernel); the group then runs in stages, one per
 * reduction it reads.  TVM keeps a reduction as the last op of its group
 * ("Fusion rules"); this flag lifts that for row reductions only. */
#define GTF_ROW_RESIDENT 2u
/* Duplicate fusion (DisCo, "Background and Motivation": the fusion
 * approaches for a predecessor with several successors; "Strategy Maker":
 * duplicating a predecessor for its other successors).  Before grouping,
 * an elementwise or broadcast op whose value would cross into other groups
 * is recomputed inside each of those readers' groups.  Ops are tried in
 * program order.  A duplication is kept when no copy's value would be
 * stored (every reader of a copy shares its group) and the plan's HBM
 * bytes (then launches) strictly drop;
 * then the scan starts over.  An op whose duplication is not kept is not
 * tried again.  Copies are ops of the plan's program
 * (fuse_plan_num_ops, fuse_plan_op_origin); their outputs are never stored,
 * so tensor ids and the caller's pointer arrays are those of the
 * descriptor. */
#define GTF_DUPLICATE 4u

typedef struct gtf_fuse_plan gtf_fuse_plan;
typedef struct gtf_bucket_plan gtf_bucket_plan;

/* Build a fusion plan from a program description (host only; no device
 * call).  Steps, in the TVM page's order: annotate each op with an
 * OpPatternKind; build the forward graph; build the post-dominator tree
 * (immediate post-dominator = least common ancestor, in the tree, of the
 * op's readers; an op whose output is a graph output or unread has none);
 * run the three fusion phases with CheckPath / CommitFuse over a
 * union-find; compile each group into an op-program.  The descriptor is
 * copied; the caller may free it afterwards.
 * Errors: GTF_E_INVALID (NULL, version, ids, order, a tmp nobody reads, an
 * in tensor written, a tensor written twice), GTF_E_UNSUPPORTED (opcode,
 * dtype, rank, u8 output), GTF_E_SHAPE (broadcast/declared shape
 * mismatch), GTF_E_LIMIT (a single op that no kernel can run).  On error
 * *out is set to NULL.
 * Diagnostics: with the environment variable GTF_TRACE set, every plan made
 * prints one line per group to stderr (its ops, domain, items, panel and
 * row-block shape, threads per row, sub-tiles, spill slots, stages). */
int fuse_plan_create(const gtf_program_desc* desc, uint32_t flags, gtf_fuse_plan** out);

/* A plan from an explicit grouping: group_of[i] (>= 0) labels descriptor
 * op i; ops with equal labels form one group.  Refused (GTF_E_INVALID, with
 * the reason) unless the group graph is acyclic, which makes every group
 * convex, and every group is within the op limit and runs as one launch
 * (argument limit, one broadcast domain, reduction stages, the kernel's
 * registers, LDS and instruction buffer).  This is how a searched or
 * hand-made plan outside the fusion rules is given to the library. */
int fuse_plan_create_grouped(const gtf_program_desc* desc, const int32_t* group_of,
                             gtf_fuse_plan** out);

/* DisCo's backtracking search over fusion plans (DisCo, "Strategy Maker";
 * strategy space of its Sec. 3.2).  A queue of candidate plans ordered by
 * cost (ties: insertion order) starts with the program unfused, every op
 * its own launch.  Each step:
 *  - dequeue the cheapest plan H;
 *  - for method (i) and then method (ii), make one candidate by applying
 *    that method to H n times, n drawn from 0..beta:
 *    - (i) non-duplicate fusion: a random op v among those with a
 *      predecessor op in another group, and a random such predecessor p;
 *      p's group merges into v's group;
 *    - (ii) duplicate fusion: the same, but when p has other readers, a copy
 *      of p joins v's group and feeds v instead;
 *    - a move whose result is not a valid plan (as fuse_plan_create_grouped
 *      checks it) is not applied;
 *  - cost each candidate once through the caller's callback;
 *  - keep it as the best when it is cheaper;
 *  - enqueue it when its cost is at most alpha times the best.
 * The search ends when the queue is empty, the best has not changed for
 * max_stall steps, or after max_steps steps (0: unbounded).  Method (iii),
 * combining AllReduce instructions, has nothing to act on with one GPU and
 * no AllReduce.
 * Random numbers come from SplitMix64 (Steele, Lea and Flood, OOPSLA 2014)
 * seeded with `seed`; draws per step: n for (i), each move's v then p, n
 * for (ii), each move's v then p.  A step without a new best counts
 * towards max_stall.
 * The callback gets a compiled candidate plan, valid only during the call
 * and runnable on the descriptor's tensors.  It returns the candidate's
 * cost, e.g. its measured time; a negative or NaN value stops the search
 * with GTF_E_INVALID.  On success *best is the best plan (destroy it with
 * fuse_plan_destroy); its program may hold copies (fuse_plan_op_origin).
 * stats may be NULL.  The page's defaults: alpha 1.05, beta 10, max_stall
 * 1000. */
typedef double (*gtf_cost_fn)(void* ctx, const gtf_fuse_plan* candidate);
typedef struct {
  double alpha;      /* >= 1 */
  int32_t beta;      /* >= 0 */
  int32_t max_stall; /* >= 1 */
  uint64_t seed;
  int32_t max_steps; /* 0: unbounded */
  int32_t reserved;
} gtf_search_params;
typedef struct {
  int64_t steps, evaluations, queue_left;
  double start_cost, best_cost;
} gtf_search_stats;
int fuse_plan_search(const gtf_program_desc* desc, const gtf_search_params* params,
                     gtf_cost_fn cost, void* ctx, gtf_fuse_plan** best,
                     gtf_search_stats* stats);

/* Number of groups; groups are numbered in an order that respects their
 * dependencies, so running 0..n-1 in order runs the program. */
int fuse_plan_num_groups(const gtf_fuse_plan* plan, int32_t* n);

/* Ops of the plan's program: the descriptor's n_ops, or more when
 * GTF_DUPLICATE added copies (and fewer originals it left unread). */
int fuse_plan_num_ops(const gtf_fuse_plan* plan, int32_t* n);

/* origin[i] = the descriptor op that program op i computes (i itself
 * without GTF_DUPLICATE).  origin holds fuse_plan_num_ops entries. */
int fuse_plan_op_origin(const gtf_fuse_plan* plan, int32_t* origin);

/* Ops of group g (ascending program op ids) and the group's OpPatternKind
 * (max over its members).  op_ids may be NULL to ask only for *n_ops;
 * otherwise it must hold cap entries (GTF_E_LIMIT if cap < *n_ops). */
int fuse_plan_group_info(const gtf_fuse_plan* plan, int32_t g, int32_t* op_ids, int32_t cap,
                         int32_t* n_ops, int32_t* pattern_kind);

/* The plan's program, in the descriptor's format: its tensors (the
 * descriptor's, then internal ones written by copies, role GTF_ROLE_TMP)
 * and its ops (topological; group_info's op ids index them).  Either array
 * may be NULL to ask only for the count; otherwise it must hold cap
 * entries (GTF_E_LIMIT if fewer). */
int fuse_plan_program(const gtf_fuse_plan* plan, gtf_tensor_desc* tensors, int32_t cap_tensors,
                      int32_t* n_tensors, gtf_op_desc* ops, int32_t cap_ops, int32_t* n_ops);

/* External tensors of group g (descriptor tensor ids): every tensor the
 * launch reads or writes in device memory, each once.  tensor_ids may be
 * NULL to ask only for *n; otherwise it must hold cap entries
 * (GTF_E_LIMIT if cap < *n). */
int fuse_plan_group_tensors(const gtf_fuse_plan* plan, int32_t g, int32_t* tensor_ids,
                            int32_t cap, int32_t* n);

/* Per-op annotation and post-dominator tree of the plan's program (both
 * arrays hold fuse_plan_num_ops entries; ipdom[i] = -1 when op i has no
 * immediate post-dominator). */
int fuse_plan_op_info(const gtf_fuse_plan* plan, int32_t* pattern_kind, int32_t* ipdom);

/* Launch shape of group g, for diagnostics and for checking the kernel's
 * address arithmetic on the host. */
typedef struct {
  int64_t rows, cols;     /* launch domain; a group with no broadcast operand
                             and no reduction runs flat as 1 x numel        */
  int64_t items;          /* work items = row blocks x column panels        */
  int32_t panels;         /* column panels (staged in LDS one at a time)    */
  int32_t rows_per_item;  /* one or two passes of 256 / threads_per_row rows */
  int32_t panel_width;    /* columns per panel, a multiple of 8             */
  int32_t threads_per_row;
  int32_t subtiles;       /* 8-element sub-tiles a lane holds per dispatched
                             instruction: 4 (wide kernel) or 1 (narrow)     */
  int32_t lds_bytes;      /* dynamic LDS per workgroup                      */
  int32_t program_length; /* op-program instructions, all phases            */
  int32_t spill_slots;    /* op-program spill slots used                    */
  int32_t spill_slots_max;/* spill slots of the kernel: 0 or 2 (wide), 6 (narrow) */
  int32_t reduce;         /* the last stage's reduction: 0 none, 1 row sum,
                             2 row mean, 3 row max; 4 mean and variance, 5
                             max and sum of exponentials (each a pair taken
                             in one pass, GTF_ROW_RESIDENT)                 */
  int32_t stages;         /* element stages: 1, or more in a group that reads
                             its own row reductions (GTF_ROW_RESIDENT)      */
  int32_t reserved;
} gtf_group_geometry;

int fuse_plan_group_geometry(const gtf_fuse_plan* plan, int32_t g, gtf_group_geometry* out);

/* The compiled op program of group g, for checking the group compiler on
 * the host: a replay of the instructions must give the group's ops'
 * results.  An instruction names one form of the executor's internal
 * instruction set (numbered in the order of the library's form
 * enumeration), its argument (a slot or register index) and an immediate.
 * The column program is instructions [0, n_col); each stage runs its row
 * program, then its element program, then ends in its reduction. */
#define GTF_MAX_STAGES 4
typedef struct {
  uint16_t form;
  uint16_t arg;
  float imm;
} gtf_instr;

typedef struct {
  int32_t row_off, row_len;    /* row program: [row_off, row_off + row_len)   */
  int32_t elem_off, elem_len;  /* element program                              */
  int32_t reduce;              /* as gtf_group_geometry.reduce (0: none)       */
  int32_t reduce_lds;          /* LDS row slot of the (first) result, or -1    */
  int32_t reduce_slot;         /* external slot of the (first) result, or -1   */
  int32_t reduce2_lds;         /* the second result of a paired reduction      */
  int32_t reduce2_slot;
} gtf_stage_code;

typedef struct {
  int32_t n_col;               /* column program length                        */
  int32_t n_stages;
  gtf_stage_code stage[GTF_MAX_STAGES];
  int32_t n_instr;             /* instructions over all phases                 */
  int32_t n_slots;             /* external slots, in fuse_plan_group_tensors
                                  order                                        */
  int32_t transposed_slot;     /* the slot the staged-transpose form reads, -1 */
  int32_t reserved;
  int64_t rstride[GTF_MAX_GROUP_ARGS]; /* element strides of each slot: the
                                          row and column phases and the
                                          addressed loads read element
                                          (r, c) at r * rstride + c * cstride */
  int64_t cstride[GTF_MAX_GROUP_ARGS];
} gtf_group_code;

/* info must not be NULL; code may be NULL to ask only for info, otherwise
 * it holds cap entries (GTF_E_LIMIT if cap < info->n_instr). */
int fuse_plan_group_code(const gtf_fuse_plan* plan, int32_t g, gtf_group_code* info,
                         gtf_instr* code, int32_t cap);

/* *yes = 1 when tensor_id must live in device memory during a run: every
 * in and out tensor, and each tmp read by a group other than its
 * producer's.  The caller allocates those; other tmps need no memory. */
int fuse_plan_is_materialized(const gtf_fuse_plan* plan, int32_t tensor_id, int32_t* yes);

/* Launch group g on the stream.  tensor_ptrs has n_tensors entries indexed
 * by tensor id; entries the group does not touch, and zero-size tensors,
 * may be NULL.  Device
 * pointers; any alignment is accepted (16-byte aligned pointers and rows
 * take the vector path).  Error: GTF_E_INVALID for a NULL pointer the group
 * needs, GTF_E_HIP when the launch fails.  Nothing is launched on error. */
int fuse_group_run(const gtf_fuse_plan* plan, int32_t g, void* const* tensor_ptrs,
                   void* hip_stream);

/* All groups, in order, on one stream (one launch per group). */
int fuse_plan_run(const gtf_fuse_plan* plan, void* const* tensor_ptrs, void* hip_stream);

void fuse_plan_destroy(gtf_fuse_plan* plan);

/* ---- one launch over many tensor sets ---------------------------------
 * Joint op and tensor fusion in one kernel (DisCo: op fusion and tensor
 * fusion chosen together; tensor fusion sends many small tensors as one):
 * group g of a plan, which must be flat (elementwise only: no broadcast
 * operand and no reduction), runs over n_sets independent sets of tensors
 * in a single launch.  Set s binds every tensor of the group to buffers of
 * numel[s] elements of their own; the plan's shapes only fix the program,
 * the dtypes and the roles.  Typical use: the elementwise epilogue of every
 * parameter gradient of a model, each set's output bound to its bucket
 * slot (bucket_plan_slot_address) with the 1/N average in the program, so
 * the epilogue and the pack are one kernel.
 * Errors: GTF_E_INVALID (NULL, bad g, n_sets < 0, numel < 0),
 * GTF_E_UNSUPPORTED (the group is not flat). */
typedef struct gtf_fuse_multi gtf_fuse_multi;
int fuse_multi_create(const gtf_fuse_plan* plan, int32_t g, int32_t n_sets, const int64_t* numel,
                      gtf_fuse_multi** out);

/* Bytes of device workspace for the run's item table, pointer table and
 * per-set alignment masks. */
int fuse_multi_workspace_bytes(const gtf_fuse_multi* m, size_t* bytes);

/* tensor_ptrs holds n_sets * n_tensors device pointers, set-major: entry
 * s * n_tensors + t is set s's buffer for tensor id t (entries the group
 * does not touch, and zero-size sets, may be NULL; any element alignment is
 * accepted).  Copies the tables into dev_workspace (caller-owned, at least
 * workspace_bytes, 16-byte aligned) asynchronously on the stream; runs read
 * them there, so bind again when a pointer changes.
 * Errors: GTF_E_INVALID (NULL, or a NULL pointer the group needs). */
int fuse_multi_bind(gtf_fuse_multi* m, void* const* tensor_ptrs, void* dev_workspace,
                    void* hip_stream);

/* One launch on the stream.  Errors: GTF_E_STATE (not bound), GTF_E_HIP. */
int fuse_multi_run(const gtf_fuse_multi* m, void* hip_stream);

void fuse_multi_destroy(gtf_fuse_multi* m);

/* ---- tensor-fusion buckets --------------------------------------------
 * Plan (host only): next-fit in the given (production) order: tensor i
 * joins the open bucket if bucket_bytes + bytes_i <= cap_bytes or the open
 * bucket is empty, else it opens a new bucket.  Offsets are dense element
 * offsets (the fused size is the sum of the sizes; no padding, no
 * splitting).  A zero-size tensor takes the open bucket's current offset.
 * dtype: GTF_F32 or GTF_BF16.  flags must be 0.
 * Errors: GTF_E_INVALID (NULL, n < 0, numel < 0, cap_bytes <= 0),
 * GTF_E_UNSUPPORTED (dtype). */
int bucket_plan_create(const int64_t* numel, int32_t n, int32_t dtype, int64_t cap_bytes,
                       uint32_t flags, gtf_bucket_plan** out);

/* Query the plan.  Any output pointer may be NULL.  bucket_of and offset
 * hold n entries, bucket_numel holds *n_buckets entries. */
int bucket_plan_query(const gtf_bucket_plan* plan, int32_t* n_buckets, int32_t* bucket_of,
                      int64_t* offset, int64_t* bucket_numel);

/* Bytes of device workspace the plan's chunk table needs. */
int bucket_plan_workspace_bytes(const gtf_bucket_plan* plan, size_t* bytes);

/* Copy the chunk table into dev_workspace (caller-owned, at least
 * workspace_bytes, 16-byte aligned) asynchronously on the stream.  Later
 * runs read it there: the caller keeps it intact and must bind again after
 * writing into it.  Runs of one plan on different streams that may overlap
 * need one plan each. */
int bucket_plan_bind(gtf_bucket_plan* plan, void* dev_workspace, void* hip_stream);

/* pack:   buckets[b][offset_i + j] = fl(src[i][j] * scale)
 * unpack: dst[i][j] = fl(buckets[b][offset_i + j] * scale)
 * with one fp32 multiply (bf16: widen, multiply, round once); scale == 1
 * copies bits unchanged.  src/dst have n entries (NULL allowed only for
 * zero-size tensors), buckets has n_buckets entries.  One launch per up to
 * 256 tensors-plus-buckets (every workload here fits in one).
 * Errors: GTF_E_STATE (not bound), GTF_E_INVALID (NULL), GTF_E_HIP. */
int bucket_pack(const gtf_bucket_plan* plan, const void* const* src, void* const* buckets,
                float scale, void* hip_stream);
int bucket_unpack(const gtf_bucket_plan* plan, const void* const* buckets, void* const* dst,
                  float scale, void* hip_stream);

/* The same plan as one launch per tensor: the per-tensor baseline the
 * single-launch path is measured against. */
int bucket_pack_per_tensor(const gtf_bucket_plan* plan, const void* const* src,
                           void* const* buckets, float scale, void* hip_stream);
int bucket_unpack_per_tensor(const gtf_bucket_plan* plan, const void* const* buckets,
                             void* const* dst, float scale, void* hip_stream);

/* bucket_pack for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it): the
 * same pack, with the plan's chunk table copied (hipMemcpyAsync from the
 * plan's host copy, on the stream) into a 1 MiB array the library holds in
 * device memory on each GPU it runs on, instead of a workspace from
 * bucket_plan_bind (which this call neither needs nor touches).  Allocates
 * nothing.  Every call on one GPU shares that array: calls that overlap on
 * one GPU race (serialize them, e.g. on one stream).  Arguments, layout and
 * results as bucket_pack.
 * Errors: GTF_E_INVALID (NULL plan or pointer arrays, NULL tensor or bucket
 * pointer of nonzero size), GTF_E_LIMIT (a chunk table over 1 MiB: more
 * than 43,690 chunks of at most 16 KiB of payload each, so at most about
 * 179M fp32 or 358M bf16 elements), GTF_E_HIP. */
int bucket_pack_static(const gtf_bucket_plan* plan, const void* const* src, void* const* buckets,
                       float scale, void* hip_stream);

/* Joint op and tensor fusion (DisCo: op fusion and tensor fusion decided
 * together; the fused tensor is the concatenation of its members).  *out =
 * the device address of tensor i's place in its bucket, buckets[bucket_of[i]]
 * + offset[i] elements.  A fused group whose output is gradient i can be run
 * with that address as the output pointer and a final mul_imm(1/N) in its
 * program: its stores then are the pack (x * scale in one fp32 multiply, as
 * bucket_pack computes), and bucket_pack is not needed for tensor i.  The
 * address is generally only 4-byte (bf16: 2-byte) aligned; the executor takes
 * element-wide accesses for such a slot.  Host arithmetic only.
 * Errors: GTF_E_INVALID (NULL plan, buckets or out; i out of range; NULL
 * bucket pointer for a tensor of nonzero size). */
int bucket_plan_slot_address(const gtf_bucket_plan* plan, void* const* buckets, int32_t i,
                             void** out);

void bucket_plan_destroy(gtf_bucket_plan* plan);

/* ---- measurement helper -------------------------------------------------
 * A plain device-to-device copy kernel (16-byte vector loads and stores):
 * the achievable-bandwidth ceiling and the reference for scaling hardware
 * byte counters.  Both pointers 16-byte aligned; nbytes a multiple of 16. */
int gtf_device_copy(void* dst, const void* src, size_t nbytes, void* hip_stream);

/* Streaming-ceiling probes: nbytes of 16-byte words moved with the knobs
 * that decide how close a streaming kernel comes to peak HBM bandwidth.
 *   kind         0 copy src -> dst, 1 read src only (each workgroup stores
 *                one 16-byte XOR of what it read at dst + 16 * workgroup),
 *                2 write dst only (src unused, may be NULL)
 *   depth        16-byte loads (or stores) in flight per thread: 4, 8, 16
 *   nontemporal  1: streaming (nontemporal) loads and stores
 *   grid_per_cu  0: one workgroup of 256 threads per 256 * depth words;
 *                k > 0: at most k workgroups per compute unit, each looping
 *                over the words with a grid stride
 * dst (and src) 16-byte aligned and nbytes bytes long (the read probe writes
 * at most that much); nbytes a multiple of 16.  Asynchronous on the stream.
 * Errors: GTF_E_INVALID (NULL, misaligned, bad kind or depth), GTF_E_HIP. */
int gtf_stream_probe(int32_t kind, int32_t depth, int32_t nontemporal, int32_t grid_per_cu,
                     void* dst, const void* src, size_t nbytes, void* hip_stream);

/* Message for the last non-OK status on this thread (never NULL). */
const char* gtf_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GTF_H */
