// capi.cpp -- the extern "C" entry points declared in include/gtf.h.
// Descriptor validation, plan ownership and error reporting live here;
// planning is in plan.cpp / bucket_plan.cpp, kernels in kernels.hip.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "gtf.h"
#include "plan.h"

struct gtf_fuse_plan {
  gtf::FusePlan p;
};
struct gtf_bucket_plan {
  gtf::BucketPlan b;
};
struct gtf_fuse_multi {
  gtf::CompiledGroup cg;
  int32_t n_tensors = 0;
  std::vector<int64_t> numel;            // per set
  std::vector<gtf::MultiItem> items;
  std::vector<unsigned char> staged;     // host copy of the bound tables
  size_t off_ptrs = 0, off_vec = 0, bytes = 0;
  void* workspace = nullptr;
};

namespace gtf {

thread_local std::string g_last_error = "no error";

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int launch_group(const CompiledGroup& cg, void* const* tensor_ptrs, hipStream_t stream);
int launch_bucket(const BucketPlan& b, const void* const* tens, void* const* bk, float scale,
                  bool unpack, bool per_tensor, hipStream_t stream);
int upload_chunks(BucketPlan& b, void* ws, hipStream_t stream);
int launch_bucket_static(const BucketPlan& b, const void* const* tens, void* const* bk, float scale,
                         hipStream_t stream);
int launch_copy(void* dst, const void* src, size_t nbytes, hipStream_t stream);
int launch_stream_probe(int kind, int depth, int nontemporal, int grid_per_cu, void* dst,
                        const void* src, size_t nbytes, hipStream_t stream);
int launch_multi(const CompiledGroup& cg, const void* ws, size_t off_ptrs, size_t off_vec,
                 int64_t n_items, hipStream_t stream);
int upload_bytes(void* dst, const void* src, size_t n, hipStream_t stream);

namespace {

int arity(int opc) {
  switch (opc) {
    case GTF_OP_COPY: case GTF_OP_EXP: case GTF_OP_TANH: case GTF_OP_SIGMOID:
    case GTF_OP_RELU: case GTF_OP_GELU: case GTF_OP_SQUARE: case GTF_OP_SQRT:
    case GTF_OP_RECIP: case GTF_OP_NEG: case GTF_OP_ADD_IMM: case GTF_OP_MUL_IMM:
    case GTF_OP_ROW_SUM: case GTF_OP_ROW_MEAN: case GTF_OP_ROW_MAX: case GTF_OP_TRANSPOSE:
    case GTF_OP_RESHAPE:
      return 1;
    case GTF_OP_ADD: case GTF_OP_SUB: case GTF_OP_MUL: case GTF_OP_DIV:
    case GTF_OP_MAX: case GTF_OP_MIN: case GTF_OP_DMUL: case GTF_OP_CONCAT: case GTF_OP_TUPLE:
      return 2;
    case GTF_OP_ADD3:
      return 3;
  }
  return -1;
}

std::string op_name(int i) { return "op " + std::to_string(i); }

int validate(const gtf_program_desc* d, FusePlan* p) {
  if (d == nullptr) return fail(GTF_E_INVALID, "desc is NULL");
  if (d->abi_version != GTF_ABI_VERSION)
    return fail(GTF_E_INVALID, "abi_version " + std::to_string(d->abi_version) + " != " +
                                   std::to_string(GTF_ABI_VERSION));
  if (d->n_tensors < 0 || d->n_ops < 0) return fail(GTF_E_INVALID, "negative count");
  if ((d->n_tensors > 0 && d->tensors == nullptr) || (d->n_ops > 0 && d->ops == nullptr))
    return fail(GTF_E_INVALID, "NULL tensor or op array");
  p->tensors.resize(d->n_tensors);
  for (int t = 0; t < d->n_tensors; ++t) {
    const gtf_tensor_desc& td = d->tensors[t];
    TensorInfo& ti = p->tensors[t];
    if (td.dtype != GTF_F32 && td.dtype != GTF_BF16 && td.dtype != GTF_U8)
      return fail(GTF_E_UNSUPPORTED, "tensor " + std::to_string(t) + ": dtype");
    if (td.rank != 1 && td.rank != 2)
      return fail(GTF_E_UNSUPPORTED, "tensor " + std::to_string(t) + ": rank must be 1 or 2");
    if (td.role != GTF_ROLE_IN && td.role != GTF_ROLE_OUT && td.role != GTF_ROLE_TMP)
      return fail(GTF_E_INVALID, "tensor " + std::to_string(t) + ": role");
    if (td.reserved != 0) return fail(GTF_E_INVALID, "tensor " + std::to_string(t) + ": reserved != 0");
    for (int k = 0; k < td.rank; ++k)
      if (td.shape[k] < 0) return fail(GTF_E_SHAPE, "tensor " + std::to_string(t) + ": negative extent");
    ti.dtype = td.dtype;
    ti.rank = td.rank;
    ti.role = td.role;
    ti.R = td.rank == 1 ? 1 : td.shape[0];
    ti.C = td.rank == 1 ? td.shape[0] : td.shape[1];
  }
  std::vector<int> writer(d->n_tensors, -1);
  std::vector<int> readers(d->n_tensors, 0);
  p->ops.resize(d->n_ops);
  for (int i = 0; i < d->n_ops; ++i) {
    const gtf_op_desc& od = d->ops[i];
    OpInfo& o = p->ops[i];
    // a concat reads two tensors, or one tuple
    const int ar = od.opcode == GTF_OP_CONCAT && od.n_in == 1 ? 1 : arity(od.opcode);
    if (ar < 0) return fail(GTF_E_UNSUPPORTED, op_name(i) + ": opcode " + std::to_string(od.opcode));
    if (od.n_in != ar) return fail(GTF_E_INVALID, op_name(i) + ": n_in does not match the opcode");
    if (od.flags & ~GTF_OPF_OPAQUE) return fail(GTF_E_INVALID, op_name(i) + ": unknown flags");
    if (od.out < 0 || od.out >= d->n_tensors) return fail(GTF_E_INVALID, op_name(i) + ": output id");
    for (int k = 0; k < ar; ++k) {
      const int t = od.in[k];
      if (t < 0 || t >= d->n_tensors) return fail(GTF_E_INVALID, op_name(i) + ": input id");
      if (p->tensors[t].role != GTF_ROLE_IN && writer[t] < 0)
        return fail(GTF_E_INVALID, op_name(i) + ": reads tensor " + std::to_string(t) +
                                       " before any op writes it (ops must be topological)");
      readers[t] += 1;
    }
    const int out = od.out;
    if (p->tensors[out].role == GTF_ROLE_IN)
      return fail(GTF_E_INVALID, op_name(i) + ": writes an input tensor");
    if (writer[out] >= 0) return fail(GTF_E_INVALID, op_name(i) + ": tensor written twice");
    if (p->tensors[out].dtype == GTF_U8)
      return fail(GTF_E_UNSUPPORTED, op_name(i) + ": u8 outputs are not supported");
    writer[out] = i;
    o.opcode = od.opcode;
    o.n_in = ar;
    for (int k = 0; k < ar; ++k) o.in[k] = od.in[k];
    o.out = out;
    o.imm = od.imm;
    o.flags = od.flags;
    // shapes
    const TensorInfo& to = p->tensors[out];
    if (od.opcode == GTF_OP_ROW_SUM || od.opcode == GTF_OP_ROW_MEAN || od.opcode == GTF_OP_ROW_MAX) {
      const TensorInfo& ti = p->tensors[od.in[0]];
      if (d->tensors[out].rank != 2 || to.R != ti.R || to.C != 1)
        return fail(GTF_E_SHAPE, op_name(i) + ": a row reduction of [R,C] is declared [R,1]");
    } else if (od.opcode == GTF_OP_TRANSPOSE) {
      const TensorInfo& ti = p->tensors[od.in[0]];
      if (ti.rank != 2 || d->tensors[out].rank != 2 || to.R != ti.C || to.C != ti.R)
        return fail(GTF_E_SHAPE, op_name(i) + ": transpose of [R,C] (rank 2) is declared [C,R]");
    } else if (od.opcode == GTF_OP_RESHAPE) {
      const TensorInfo& ti = p->tensors[od.in[0]];
      if (ti.R * ti.C != to.R * to.C)
        return fail(GTF_E_SHAPE, op_name(i) + ": reshape changes the element count");
    } else if (od.opcode == GTF_OP_CONCAT && ar == 1) {
      const TensorInfo& ti = p->tensors[od.in[0]];
      const int w = writer[od.in[0]];
      if (w < 0 || p->ops[w].opcode != GTF_OP_TUPLE)
        return fail(GTF_E_INVALID, op_name(i) + ": a concat of one operand reads a tuple");
      if (to.R != ti.R || to.C != ti.C || d->tensors[out].rank != 2 || to.dtype != ti.dtype)
        return fail(GTF_E_SHAPE, op_name(i) + ": a concat of a tuple is declared as the tuple");
    } else if (od.opcode == GTF_OP_CONCAT || od.opcode == GTF_OP_TUPLE) {
      const TensorInfo& a = p->tensors[od.in[0]];
      const TensorInfo& b = p->tensors[od.in[1]];
      if (a.rank != 2 || b.rank != 2 || d->tensors[out].rank != 2 || a.R != b.R || to.R != a.R ||
          a.C < 1 || b.C < 1 || to.C != a.C + b.C)
        return fail(GTF_E_SHAPE, op_name(i) + ": concat of [R,C1], [R,C2] (rank 2, C1, C2 >= 1) "
                                              "is declared [R,C1+C2]");
      if (a.dtype != b.dtype || to.dtype != a.dtype)
        return fail(GTF_E_UNSUPPORTED, op_name(i) + ": concat or tuple of two dtypes");
    } else {
      // NumPy broadcasting per axis: extents of 1 stretch to the other one
      int64_t R = 1, C = 1;
      for (int k = 0; k < ar; ++k) {
        if (p->tensors[od.in[k]].R != 1) R = p->tensors[od.in[k]].R;
        if (p->tensors[od.in[k]].C != 1) C = p->tensors[od.in[k]].C;
      }
      for (int k = 0; k < ar; ++k) {
        const TensorInfo& ti = p->tensors[od.in[k]];
        if ((ti.R != 1 && ti.R != R) || (ti.C != 1 && ti.C != C))
          return fail(GTF_E_SHAPE, op_name(i) + ": operand shapes do not broadcast");
      }
      if (to.R != R || to.C != C)
        return fail(GTF_E_SHAPE, op_name(i) + ": declared output shape differs from the result");
    }
  }
  for (int t = 0; t < d->n_tensors; ++t) {
    const int role = p->tensors[t].role;
    if (role != GTF_ROLE_IN && writer[t] < 0)
      return fail(GTF_E_INVALID, "tensor " + std::to_string(t) + ": no op writes it");
    if (role == GTF_ROLE_TMP && readers[t] == 0)
      return fail(GTF_E_INVALID, "tensor " + std::to_string(t) + ": tmp that no op reads");
  }
  // a tuple is read only by concats of one operand, and is not a graph output
  for (int i = 0; i < d->n_ops; ++i) {
    if (p->ops[i].opcode != GTF_OP_TUPLE) continue;
    const int t = p->ops[i].out;
    if (p->tensors[t].role != GTF_ROLE_TMP)
      return fail(GTF_E_INVALID, op_name(i) + ": a tuple is not a graph output");
    for (int j = 0; j < d->n_ops; ++j)
      for (int k = 0; k < p->ops[j].n_in; ++k)
        if (p->ops[j].in[k] == t && !(p->ops[j].opcode == GTF_OP_CONCAT && p->ops[j].n_in == 1))
          return fail(GTF_E_INVALID, op_name(j) + ": a tuple is read only by a concat of it");
  }
  return GTF_OK;
}

}  // namespace
}  // namespace gtf

using namespace gtf;

extern "C" {

const char* gtf_last_error(void) { return g_last_error.c_str(); }

int fuse_plan_create(const gtf_program_desc* desc, uint32_t flags, gtf_fuse_plan** out) {
  if (out == nullptr) return fail(GTF_E_INVALID, "out is NULL");
  *out = nullptr;
  if (flags & ~(GTF_NO_FUSE | GTF_ROW_RESIDENT | GTF_DUPLICATE))
    return fail(GTF_E_INVALID, "unknown flags");
  gtf_fuse_plan* h = new (std::nothrow) gtf_fuse_plan();
  if (h == nullptr) return fail(GTF_E_LIMIT, "out of host memory");
  int st = validate(desc, &h->p);
  if (st == GTF_OK)
    st = build_fuse_plan(&h->p, (flags & GTF_NO_FUSE) == 0, (flags & GTF_ROW_RESIDENT) != 0,
                         (flags & GTF_DUPLICATE) != 0);
  if (st != GTF_OK) {
    delete h;
    return st;
  }
  *out = h;
  return GTF_OK;
}

int fuse_plan_create_grouped(const gtf_program_desc* desc, const int32_t* group_of,
                             gtf_fuse_plan** out) {
  if (out == nullptr) return fail(GTF_E_INVALID, "out is NULL");
  *out = nullptr;
  gtf_fuse_plan* h = new (std::nothrow) gtf_fuse_plan();
  if (h == nullptr) return fail(GTF_E_LIMIT, "out of host memory");
  int st = validate(desc, &h->p);
  if (st == GTF_OK && group_of == nullptr && !h->p.ops.empty())
    st = fail(GTF_E_INVALID, "group_of is NULL");
  if (st == GTF_OK) {
    std::vector<int> labels(group_of, group_of + h->p.ops.size());
    st = build_grouped_plan(&h->p, labels);
  }
  if (st != GTF_OK) {
    delete h;
    return st;
  }
  *out = h;
  return GTF_OK;
}

int fuse_plan_search(const gtf_program_desc* desc, const gtf_search_params* params,
                     gtf_cost_fn cost, void* ctx, gtf_fuse_plan** best,
                     gtf_search_stats* stats) {
  if (best == nullptr || params == nullptr || cost == nullptr)
    return fail(GTF_E_INVALID, "NULL argument");
  *best = nullptr;
  gtf_fuse_plan* h = new (std::nothrow) gtf_fuse_plan();
  if (h == nullptr) return fail(GTF_E_LIMIT, "out of host memory");
  int st = validate(desc, &h->p);
  if (st == GTF_OK) {
    SearchParams prm;
    prm.alpha = params->alpha;
    prm.beta = params->beta;
    prm.max_stall = params->max_stall;
    prm.seed = params->seed;
    prm.max_steps = params->max_steps;
    SearchStats ss;
    gtf_fuse_plan cand;
    st = search_plan(&h->p, prm,
                     [&](const FusePlan& fp) {
                       cand.p = fp;
                       return cost(ctx, &cand);
                     },
                     &ss);
    if (st == GTF_OK && stats) {
      stats->steps = ss.steps;
      stats->evaluations = ss.evaluations;
      stats->queue_left = ss.queue_left;
      stats->start_cost = ss.start_cost;
      stats->best_cost = ss.best_cost;
    }
  }
  if (st != GTF_OK) {
    delete h;
    return st;
  }
  *best = h;
  return GTF_OK;
}

int fuse_plan_num_groups(const gtf_fuse_plan* plan, int32_t* n) {
  if (plan == nullptr || n == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  *n = (int32_t)plan->p.groups.size();
  return GTF_OK;
}

int fuse_plan_num_ops(const gtf_fuse_plan* plan, int32_t* n) {
  if (plan == nullptr || n == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  *n = (int32_t)plan->p.ops.size();
  return GTF_OK;
}

int fuse_plan_op_origin(const gtf_fuse_plan* plan, int32_t* origin) {
  if (plan == nullptr || origin == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  for (size_t i = 0; i < plan->p.ops.size(); ++i) origin[i] = plan->p.origin[i];
  return GTF_OK;
}

int fuse_plan_group_info(const gtf_fuse_plan* plan, int32_t g, int32_t* op_ids, int32_t cap,
                         int32_t* n_ops, int32_t* pattern_kind) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(GTF_E_INVALID, "group index");
  const Group& G = plan->p.groups[g];
  if (n_ops) *n_ops = (int32_t)G.ops.size();
  if (pattern_kind) *pattern_kind = G.pattern;
  if (op_ids) {
    if (cap < (int32_t)G.ops.size()) return fail(GTF_E_LIMIT, "op_ids capacity too small");
    for (size_t k = 0; k < G.ops.size(); ++k) op_ids[k] = G.ops[k];
  }
  return GTF_OK;
}

int fuse_plan_program(const gtf_fuse_plan* plan, gtf_tensor_desc* tensors, int32_t cap_tensors,
                      int32_t* n_tensors, gtf_op_desc* ops, int32_t cap_ops, int32_t* n_ops) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  const FusePlan& p = plan->p;
  if (n_tensors) *n_tensors = (int32_t)p.tensors.size();
  if (n_ops) *n_ops = (int32_t)p.ops.size();
  if (tensors) {
    if (cap_tensors < (int32_t)p.tensors.size()) return fail(GTF_E_LIMIT, "tensor capacity too small");
    for (size_t t = 0; t < p.tensors.size(); ++t) {
      const TensorInfo& ti = p.tensors[t];
      gtf_tensor_desc& d = tensors[t];
      d.dtype = ti.dtype;
      d.rank = ti.rank;
      d.shape[0] = ti.rank == 1 ? ti.C : ti.R;
      d.shape[1] = ti.rank == 1 ? 0 : ti.C;
      d.role = ti.role;
      d.reserved = 0;
    }
  }
  if (ops) {
    if (cap_ops < (int32_t)p.ops.size()) return fail(GTF_E_LIMIT, "op capacity too small");
    for (size_t i = 0; i < p.ops.size(); ++i) {
      const OpInfo& o = p.ops[i];
      gtf_op_desc& d = ops[i];
      d.opcode = o.opcode;
      d.n_in = o.n_in;
      for (int k = 0; k < 3; ++k) d.in[k] = k < o.n_in ? o.in[k] : 0;
      d.out = o.out;
      d.imm = o.imm;
      d.flags = o.flags;
    }
  }
  return GTF_OK;
}

int fuse_plan_group_tensors(const gtf_fuse_plan* plan, int32_t g, int32_t* tensor_ids,
                            int32_t cap, int32_t* n) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(GTF_E_INVALID, "group index");
  const std::vector<int>& st = plan->p.groups[g].code.slot_tensor;
  if (n) *n = (int32_t)st.size();
  if (tensor_ids) {
    if (cap < (int32_t)st.size()) return fail(GTF_E_LIMIT, "tensor_ids capacity too small");
    for (size_t k = 0; k < st.size(); ++k) tensor_ids[k] = st[k];
  }
  return GTF_OK;
}

int fuse_plan_op_info(const gtf_fuse_plan* plan, int32_t* pattern_kind, int32_t* ipdom) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  for (size_t i = 0; i < plan->p.ops.size(); ++i) {
    if (pattern_kind) pattern_kind[i] = plan->p.ops[i].pattern;
    if (ipdom) ipdom[i] = plan->p.ipdom[i];
  }
  return GTF_OK;
}

int fuse_plan_group_geometry(const gtf_fuse_plan* plan, int32_t g, gtf_group_geometry* out) {
  if (plan == nullptr || out == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(GTF_E_INVALID, "group index");
  const CompiledGroup& cg = plan->p.groups[g].code;
  const ExecArgs& a = cg.args;
  out->rows = a.R;
  out->cols = a.C;
  out->items = a.n_items;
  out->panels = a.n_panels;
  out->rows_per_item = a.RB;
  out->panel_width = a.PW;
  out->threads_per_row = 1 << a.tpr_log2;
  out->subtiles = a.K;
  out->lds_bytes = cg.lds_bytes;
  out->program_length = a.stage[a.n_stages - 1].el_off + a.stage[a.n_stages - 1].el_len;
  out->spill_slots = cg.max_depth;
  out->spill_slots_max = a.NS;
  out->reduce = 0;
  for (int st = 0; st < a.n_stages; ++st)
    if (a.stage[st].red) out->reduce = a.stage[st].red;
  out->stages = a.n_stages;
  return GTF_OK;
}

static_assert(GTF_MAX_STAGES == kMaxStages && GTF_MAX_GROUP_ARGS == kMaxSlots,
              "the program view's array sizes are the executor's");
static_assert(sizeof(gtf_instr) == sizeof(Instr), "gtf_instr mirrors Instr");

int fuse_plan_group_code(const gtf_fuse_plan* plan, int32_t g, gtf_group_code* info,
                         gtf_instr* code, int32_t cap) {
  if (plan == nullptr || info == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(GTF_E_INVALID, "group index");
  const CompiledGroup& cg = plan->p.groups[g].code;
  const ExecArgs& a = cg.args;
  std::memset(info, 0, sizeof(*info));
  info->n_col = a.n_col;
  info->n_stages = a.n_stages;
  for (int st = 0; st < a.n_stages; ++st) {
    const StageDesc& S = a.stage[st];
    gtf_stage_code& o = info->stage[st];
    o.row_off = S.row_off;
    o.row_len = S.row_len;
    o.elem_off = S.el_off;
    o.elem_len = S.el_len;
    o.reduce = S.red;
    o.reduce_lds = S.red_lds;
    o.reduce_slot = S.red_slot;
    o.reduce2_lds = S.red >= 4 ? S.red2_lds : -1;
    o.reduce2_slot = S.red >= 4 ? S.red2_slot : -1;
  }
  info->n_instr = a.stage[a.n_stages - 1].el_off + a.stage[a.n_stages - 1].el_len;
  info->n_slots = (int32_t)cg.slot_tensor.size();
  info->transposed_slot = a.n_tr > 0 ? a.tr_slot : -1;
  for (int s = 0; s < kMaxSlots; ++s) {
    info->rstride[s] = a.rstride[s];
    info->cstride[s] = a.cstride[s];
  }
  if (code == nullptr) return GTF_OK;
  if (cap < info->n_instr) return fail(GTF_E_LIMIT, "code capacity too small");
  for (int i = 0; i < info->n_instr; ++i) {
    code[i].form = a.prog[i].code;
    code[i].arg = a.prog[i].arg;
    code[i].imm = a.prog[i].imm;
  }
  return GTF_OK;
}

int fuse_plan_is_materialized(const gtf_fuse_plan* plan, int32_t tensor_id, int32_t* yes) {
  if (plan == nullptr || yes == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  if (tensor_id < 0 || tensor_id >= (int32_t)plan->p.n_desc_tensors)
    return fail(GTF_E_INVALID, "tensor id");
  *yes = plan->p.materialized[tensor_id] ? 1 : 0;
  return GTF_OK;
}

int fuse_group_run(const gtf_fuse_plan* plan, int32_t g, void* const* tensor_ptrs, void* hip_stream) {
  if (plan == nullptr || tensor_ptrs == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(GTF_E_INVALID, "group index");
  return launch_group(plan->p.groups[g].code, tensor_ptrs, (hipStream_t)hip_stream);
}

int fuse_plan_run(const gtf_fuse_plan* plan, void* const* tensor_ptrs, void* hip_stream) {
  if (plan == nullptr || tensor_ptrs == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  // check every pointer first so nothing is launched on error
  for (const Group& G : plan->p.groups)
    for (size_t s = 0; s < G.code.slot_tensor.size(); ++s)
      if (tensor_ptrs[G.code.slot_tensor[s]] == nullptr && G.code.slot_numel[s] > 0)
        return fail(GTF_E_INVALID, "tensor " + std::to_string(G.code.slot_tensor[s]) +
                                       " has no device pointer");
  for (const Group& G : plan->p.groups) {
    int st = launch_group(G.code, tensor_ptrs, (hipStream_t)hip_stream);
    if (st != GTF_OK) return st;
  }
  return GTF_OK;
}

void fuse_plan_destroy(gtf_fuse_plan* plan) { delete plan; }

int bucket_plan_create(const int64_t* numel, int32_t n, int32_t dtype, int64_t cap_bytes,
                       uint32_t flags, gtf_bucket_plan** out) {
  if (out == nullptr) return fail(GTF_E_INVALID, "out is NULL");
  *out = nullptr;
  if (n < 0 || (n > 0 && numel == nullptr)) return fail(GTF_E_INVALID, "numel");
  if (cap_bytes <= 0) return fail(GTF_E_INVALID, "cap_bytes must be positive");
  if (flags != 0) return fail(GTF_E_INVALID, "flags must be 0");
  if (dtype != GTF_F32 && dtype != GTF_BF16) return fail(GTF_E_UNSUPPORTED, "bucket dtype");
  for (int i = 0; i < n; ++i)
    if (numel[i] < 0) return fail(GTF_E_INVALID, "negative numel");
  gtf_bucket_plan* h = new (std::nothrow) gtf_bucket_plan();
  if (h == nullptr) return fail(GTF_E_LIMIT, "out of host memory");
  h->b.dtype = dtype;
  h->b.cap_bytes = cap_bytes;
  h->b.numel.assign(numel, numel + n);
  int st = build_bucket_plan(&h->b);
  if (st != GTF_OK) {
    delete h;
    return st;
  }
  *out = h;
  return GTF_OK;
}

int bucket_plan_query(const gtf_bucket_plan* plan, int32_t* n_buckets, int32_t* bucket_of,
                      int64_t* offset, int64_t* bucket_numel) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  const BucketPlan& b = plan->b;
  if (n_buckets) *n_buckets = (int32_t)b.bucket_numel.size();
  for (size_t i = 0; i < b.numel.size(); ++i) {
    if (bucket_of) bucket_of[i] = b.bucket_of[i];
    if (offset) offset[i] = b.offset[i];
  }
  if (bucket_numel)
    for (size_t k = 0; k < b.bucket_numel.size(); ++k) bucket_numel[k] = b.bucket_numel[k];
  return GTF_OK;
}

int bucket_plan_workspace_bytes(const gtf_bucket_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  *bytes = plan->b.chunks.size() * sizeof(Chunk);
  return GTF_OK;
}

int bucket_plan_bind(gtf_bucket_plan* plan, void* dev_workspace, void* hip_stream) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  if (dev_workspace == nullptr && !plan->b.chunks.empty())
    return fail(GTF_E_INVALID, "workspace is NULL");
  if (((uintptr_t)dev_workspace & 15) != 0) return fail(GTF_E_INVALID, "workspace not 16-byte aligned");
  return upload_chunks(plan->b, dev_workspace, (hipStream_t)hip_stream);
}

static int bucket_run(const gtf_bucket_plan* plan, const void* const* tens, void* const* bk,
                      float scale, bool unpack, bool per_tensor, void* hip_stream) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  const BucketPlan& b = plan->b;
  if (b.numel.empty()) return GTF_OK;
  if (tens == nullptr || bk == nullptr) return fail(GTF_E_INVALID, "NULL pointer array");
  if (b.workspace == nullptr && !b.chunks.empty())
    return fail(GTF_E_STATE, "bucket plan used before bucket_plan_bind");
  return launch_bucket(b, tens, bk, scale, unpack, per_tensor, (hipStream_t)hip_stream);
}

int bucket_pack(const gtf_bucket_plan* plan, const void* const* src, void* const* buckets,
                float scale, void* hip_stream) {
  return bucket_run(plan, src, buckets, scale, false, false, hip_stream);
}

int bucket_unpack(const gtf_bucket_plan* plan, const void* const* buckets, void* const* dst,
                  float scale, void* hip_stream) {
  return bucket_run(plan, (const void* const*)dst, (void* const*)buckets, scale, true, false,
                    hip_stream);
}

int bucket_pack_per_tensor(const gtf_bucket_plan* plan, const void* const* src,
                           void* const* buckets, float scale, void* hip_stream) {
  return bucket_run(plan, src, buckets, scale, false, true, hip_stream);
}

int bucket_pack_static(const gtf_bucket_plan* plan, const void* const* src, void* const* buckets,
                       float scale, void* hip_stream) {
  if (plan == nullptr) return fail(GTF_E_INVALID, "plan is NULL");
  const BucketPlan& b = plan->b;
  if (b.numel.empty()) return GTF_OK;
  if (src == nullptr || buckets == nullptr) return fail(GTF_E_INVALID, "NULL pointer array");
  return launch_bucket_static(b, src, buckets, scale, (hipStream_t)hip_stream);
}

int bucket_unpack_per_tensor(const gtf_bucket_plan* plan, const void* const* buckets,
                             void* const* dst, float scale, void* hip_stream) {
  return bucket_run(plan, (const void* const*)dst, (void* const*)buckets, scale, true, true,
                    hip_stream);
}

int bucket_plan_slot_address(const gtf_bucket_plan* plan, void* const* buckets, int32_t i,
                             void** out) {
  if (plan == nullptr || buckets == nullptr || out == nullptr)
    return fail(GTF_E_INVALID, "NULL argument");
  const BucketPlan& b = plan->b;
  if (i < 0 || i >= (int32_t)b.numel.size()) return fail(GTF_E_INVALID, "tensor index");
  char* base = (char*)buckets[b.bucket_of[i]];
  if (base == nullptr && b.numel[i] > 0) return fail(GTF_E_INVALID, "bucket pointer is NULL");
  const int64_t elem = b.dtype == GTF_BF16 ? 2 : 4;
  *out = base == nullptr ? nullptr : base + b.offset[i] * elem;
  return GTF_OK;
}

void bucket_plan_destroy(gtf_bucket_plan* plan) { delete plan; }

int fuse_multi_create(const gtf_fuse_plan* plan, int32_t g, int32_t n_sets, const int64_t* numel,
                      gtf_fuse_multi** out) {
  if (plan == nullptr || out == nullptr || (numel == nullptr && n_sets > 0))
    return fail(GTF_E_INVALID, "NULL argument");
  if (g < 0 || g >= (int32_t)plan->p.groups.size()) return fail(GTF_E_INVALID, "group index");
  if (n_sets < 0) return fail(GTF_E_INVALID, "n_sets < 0");
  const CompiledGroup& cg = plan->p.groups[g].code;
  const ExecArgs& a = cg.args;
  if (a.R > 1 || a.n_col > 0 || a.n_stages != 1 || a.stage[0].row_len > 0 || a.stage[0].red != 0)
    return fail(GTF_E_UNSUPPORTED, "group is not flat (broadcast operand or reduction)");
  for (int32_t s = 0; s < n_sets; ++s)
    if (numel[s] < 0) return fail(GTF_E_INVALID, "numel < 0");
  gtf_fuse_multi* m = new (std::nothrow) gtf_fuse_multi;
  if (m == nullptr) return fail(GTF_E_INVALID, "out of host memory");
  m->cg = cg;
  m->n_tensors = (int32_t)plan->p.n_desc_tensors;
  m->numel.assign(numel, numel + n_sets);
  for (int32_t s = 0; s < n_sets; ++s)
    for (int64_t off = 0; off < numel[s]; off += a.PW) {
      MultiItem it;
      it.off = off;
      it.n = (int32_t)std::min<int64_t>(a.PW, numel[s] - off);
      it.set = s;
      m->items.push_back(it);
    }
  auto up16 = [](size_t x) { return (x + 15) / 16 * 16; };
  m->off_ptrs = up16(m->items.size() * sizeof(MultiItem));
  m->off_vec = up16(m->off_ptrs + (size_t)n_sets * cg.n_slots * sizeof(void*));
  m->bytes = up16(m->off_vec + (size_t)n_sets * sizeof(uint32_t));
  *out = m;
  return GTF_OK;
}

int fuse_multi_workspace_bytes(const gtf_fuse_multi* m, size_t* bytes) {
  if (m == nullptr || bytes == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  *bytes = m->bytes;
  return GTF_OK;
}

int fuse_multi_bind(gtf_fuse_multi* m, void* const* tensor_ptrs, void* dev_workspace,
                    void* hip_stream) {
  if (m == nullptr || dev_workspace == nullptr || (tensor_ptrs == nullptr && !m->numel.empty()))
    return fail(GTF_E_INVALID, "NULL argument");
  if (((uintptr_t)dev_workspace & 15) != 0) return fail(GTF_E_INVALID, "workspace not 16-byte aligned");
  const CompiledGroup& cg = m->cg;
  const size_t n_sets = m->numel.size();
  std::vector<unsigned char> st(m->bytes, 0);
  std::memcpy(st.data(), m->items.data(), m->items.size() * sizeof(MultiItem));
  void** ptrs = (void**)(st.data() + m->off_ptrs);
  uint32_t* vec = (uint32_t*)(st.data() + m->off_vec);
  for (size_t s = 0; s < n_sets; ++s) {
    uint32_t mask = 0;
    for (int k = 0; k < cg.n_slots; ++k) {
      void* p = tensor_ptrs[s * m->n_tensors + cg.slot_tensor[k]];
      if (p == nullptr && m->numel[s] > 0)
        return fail(GTF_E_INVALID, "set " + std::to_string(s) + ": tensor " +
                                       std::to_string(cg.slot_tensor[k]) + " has no device pointer");
      ptrs[s * cg.n_slots + k] = p;
      const uintptr_t align = cg.slot_dtype[k] == GTF_U8 ? 8 : 16;
      if (((uintptr_t)p % align) == 0) mask |= 1u << k;
    }
    vec[s] = mask;
  }
  m->staged.swap(st);
  int rc = upload_bytes(dev_workspace, m->staged.data(), m->bytes, (hipStream_t)hip_stream);
  if (rc != GTF_OK) return rc;
  m->workspace = dev_workspace;
  return GTF_OK;
}

int fuse_multi_run(const gtf_fuse_multi* m, void* hip_stream) {
  if (m == nullptr) return fail(GTF_E_INVALID, "NULL argument");
  if (m->workspace == nullptr) return fail(GTF_E_STATE, "fuse_multi_bind has not been called");
  return launch_multi(m->cg, m->workspace, m->off_ptrs, m->off_vec, (int64_t)m->items.size(),
                      (hipStream_t)hip_stream);
}

void fuse_multi_destroy(gtf_fuse_multi* m) { delete m; }

int gtf_device_copy(void* dst, const void* src, size_t nbytes, void* hip_stream) {
  if (dst == nullptr || src == nullptr) return fail(GTF_E_INVALID, "NULL pointer");
  if ((((uintptr_t)dst | (uintptr_t)src) & 15) != 0 || (nbytes & 15) != 0)
    return fail(GTF_E_INVALID, "copy needs 16-byte aligned pointers and size");
  return launch_copy(dst, src, nbytes, (hipStream_t)hip_stream);
}

int gtf_stream_probe(int32_t kind, int32_t depth, int32_t nontemporal, int32_t grid_per_cu,
                     void* dst, const void* src, size_t nbytes, void* hip_stream) {
  if (dst == nullptr || (kind != 2 && src == nullptr)) return fail(GTF_E_INVALID, "NULL pointer");
  if ((((uintptr_t)dst | (uintptr_t)src) & 15) != 0 || (nbytes & 15) != 0)
    return fail(GTF_E_INVALID, "stream probe needs 16-byte aligned pointers and size");
  return launch_stream_probe(kind, depth, nontemporal, grid_per_cu, dst, src, nbytes,
                             (hipStream_t)hip_stream);
}

}  // extern "C"
