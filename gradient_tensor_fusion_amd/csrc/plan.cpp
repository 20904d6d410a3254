// plan.cpp -- fusion planning on the host: OpPatternKind annotation, the
// forward graph, the post-dominator tree, the three-phase grouping with
// CheckPath / CommitFuse over a union-find, and group compilation.
//
// The grouping follows Apache TVM, "Operator Fusion" (docs/arch/fusion.rst):
// "Operator Pattern Classification" (the kinds and CombinePattern = max),
// "Algorithm" steps 1-4 and "Fusion rules" (the three phases, reductions
// are sinks only, opaque ops are barriers, at most kMaxFusedOps = 256 ops
// and a bounded argument count per group).  A tuple (kTuple) fuses into the
// injective concat after it in phase 1; its fields join it in phase 2.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <queue>
#include <set>
#include <string>
#include <vector>

#include "gtf.h"
#include "plan.h"

namespace gtf {

namespace {

bool is_reduce(int opc) {
  return opc == GTF_OP_ROW_SUM || opc == GTF_OP_ROW_MEAN || opc == GTF_OP_ROW_MAX;
}

// ---------------------------------------------------------------- union-find
struct UnionFind {
  std::vector<int> parent, pat, size;
  explicit UnionFind(const std::vector<int>& pats)
      : parent(pats.size()), pat(pats), size(pats.size(), 1) {
    for (size_t i = 0; i < parent.size(); ++i) parent[i] = (int)i;
  }
  int find(int x) {
    while (parent[x] != x) {
      parent[x] = parent[parent[x]];
      x = parent[x];
    }
    return x;
  }
  // merge x's set into target's set; the target's root stays the root
  void merge_into(int x, int target) {
    int rx = find(x), rt = find(target);
    if (rx == rt) return;
    parent[rx] = rt;
    // CombinePattern; a tuple fused into the group after it is an injective
    // member there
    pat[rt] = std::max(pat[rt], pat[rx] == GTF_PAT_TUPLE ? (int)GTF_PAT_INJECTIVE : pat[rx]);
    size[rt] += size[rx];
  }
};

std::vector<std::vector<int>> readers_of(const FusePlan& p) {
  std::vector<int> producer(p.tensors.size(), -1);
  for (size_t i = 0; i < p.ops.size(); ++i) producer[p.ops[i].out] = (int)i;
  std::vector<std::vector<int>> rd(p.ops.size());
  for (size_t j = 0; j < p.ops.size(); ++j) {
    const OpInfo& o = p.ops[j];
    for (int k = 0; k < o.n_in; ++k) {
      int pr = producer[o.in[k]];
      if (pr >= 0 && (rd[pr].empty() || rd[pr].back() != (int)j)) rd[pr].push_back((int)j);
    }
  }
  return rd;
}

// Post-dominator tree (Algorithm step 2): visit ops in reverse topological
// order; an op's parent is the least common ancestor, in the tree built so
// far, of all ops that read its output.  An op whose output is a graph
// output, or has no reader, hangs off the virtual root (-1).
std::vector<int> postdom_tree(const FusePlan& p, const std::vector<std::vector<int>>& rd) {
  int n = (int)p.ops.size();
  std::vector<int> parent(n, -1), depth(n, 1);
  auto dep = [&](int v) { return v < 0 ? 0 : depth[v]; };
  auto lca = [&](int a, int b) {
    while (a != b) {
      if (dep(a) >= dep(b))
        a = parent[a];  // a >= 0 here: depth 0 is only the root
      else
        b = parent[b];
    }
    return a;
  };
  for (int i = n - 1; i >= 0; --i) {
    const OpInfo& o = p.ops[i];
    if (p.tensors[o.out].role == GTF_ROLE_OUT || rd[i].empty()) {
      parent[i] = -1;
      depth[i] = 1;
      continue;
    }
    int l = rd[i][0];
    for (size_t k = 1; k < rd[i].size() && l >= 0; ++k) l = lca(l, rd[i][k]);
    parent[i] = l;
    depth[i] = dep(l) + 1;
  }
  return parent;
}

// External tensors of a member set: inputs read from outside plus outputs
// needed outside (graph outputs or read by non-members).
int count_args(const FusePlan& p, const std::vector<char>& in_set) {
  std::set<int> produced, ext;
  for (size_t i = 0; i < p.ops.size(); ++i)
    if (in_set[i]) produced.insert(p.ops[i].out);
  for (size_t i = 0; i < p.ops.size(); ++i) {
    const OpInfo& o = p.ops[i];
    for (int k = 0; k < o.n_in; ++k) {
      bool inside = produced.count(o.in[k]) != 0;
      if (in_set[i] && !inside) ext.insert(o.in[k]);
      if (!in_set[i] && inside) ext.insert(o.in[k]);
    }
  }
  for (int t : produced)
    if (p.tensors[t].role == GTF_ROLE_OUT) ext.insert(t);
  return (int)ext.size();
}

}  // namespace

// ============================================================== compilation
namespace {

enum Cls { CLS_E = 0, CLS_ROW = 1, CLS_COL = 2 };
constexpr int kNoValue = -1;

struct MOp {
  int kind;    // 0 unary form, 1 binary op, 2 imm op (slot op imm), 3 reduce, 4 copy,
               // 5 addressed load (transpose / reshape / concat of tensors in memory)
  int form;    // F_* for unary, F_ADD..F_MIN for binary, XOp for imm
  int in[2] = {-1, -1};
  int out = -1;
  float imm = 0.f;
  bool commutative = false;
  int gkind = 0;           // kind 5: 0 plain load, 1 strided gather, 2 concat of two slots
  int src[2] = {-1, -1};   // kind 5: the tensors read from memory
};

// register operands of a micro-op
int mop_arity(const MOp& m) { return m.kind == 1 ? 2 : m.kind == 5 ? 0 : 1; }

// ops that run as addressed loads of tensors in memory: transpose, reshape,
// a concat of two tensors and a tuple (a tuple's value is its fields side
// by side; a concat of one tuple is a copy of it)
bool is_gather(const OpInfo& o) {
  return o.opcode == GTF_OP_TRANSPOSE || o.opcode == GTF_OP_RESHAPE || o.opcode == GTF_OP_TUPLE ||
         (o.opcode == GTF_OP_CONCAT && o.n_in == 2);
}
bool is_join(const OpInfo& o) {
  return o.opcode == GTF_OP_TUPLE || (o.opcode == GTF_OP_CONCAT && o.n_in == 2);
}

int unary_form(int opc) {
  switch (opc) {
    case GTF_OP_EXP: return F_EXP;
    case GTF_OP_TANH: return F_TANH;
    case GTF_OP_SIGMOID: return F_SIGMOID;
    case GTF_OP_RELU: return F_RELU;
    case GTF_OP_GELU: return F_GELU;
    case GTF_OP_SQUARE: return F_SQUARE;
    case GTF_OP_SQRT: return F_SQRT;
    case GTF_OP_RECIP: return F_RECIP;
    case GTF_OP_NEG: return F_NEG;
  }
  return -1;
}

int binary_form(int opc) {
  switch (opc) {
    case GTF_OP_ADD: return F_ADD;
    case GTF_OP_SUB: return F_SUB;
    case GTF_OP_MUL: return F_MUL;
    case GTF_OP_DIV: return F_DIV;
    case GTF_OP_MAX: return F_MAX;
    case GTF_OP_MIN: return F_MIN;
  }
  return -1;
}

// x-op for "stack (op) X" and for "X (op) stack"
int xop_of(int binform, bool x_on_left) {
  switch (binform) {
    case F_ADD: return X_ADD;
    case F_MUL: return X_MUL;
    case F_MAX: return X_MAX;
    case F_MIN: return X_MIN;
    case F_SUB: return x_on_left ? X_RSUB : X_SUB;
    case F_DIV: return x_on_left ? X_RDIV : X_DIV;
  }
  return -1;
}

bool commutative(int binform) {
  return binform == F_ADD || binform == F_MUL || binform == F_MAX || binform == F_MIN;
}

// Register allocation for the A/B machine.  Values are tensor ids (>= 0) or
// synthetic temporaries (<= -2).  A value lives in any of A, B and the
// spill slots; it is spilled only when the register it sits in is about to
// be overwritten while it still has readers.
struct Codegen {
  const FusePlan& p;
  std::vector<Instr>* out;
  int phase;  // CLS_E / CLS_ROW / CLS_COL
  std::map<int, int> uses;       // remaining reads in this phase
  std::set<int> loadable;        // external tensors this phase loads
  std::map<int, int> ext_slot;   // tensor -> external slot
  std::map<int, int> lds_slot;   // value -> LDS slot (values read via X)
  std::map<int, int> xcls;       // value -> CLS_ROW / CLS_COL for X operands
  static constexpr int kEmpty = -1000000;
  enum { RA = 0, RB = 1 };       // register ids: 0 = A, 1 = B, 2.. = spill slots
  int reg[2 + kNS];
  int ns = kNS;                  // spill slots of the kernel instance
  int max_live = 0;
  bool ok = true;
  std::string why;

  void init() {
    for (int& r : reg) r = kEmpty;
  }
  void emit(int form, int arg = 0, float imm = 0.f) {
    Instr ins;
    ins.code = (uint16_t)form;
    ins.arg = (uint16_t)arg;
    ins.imm = imm;
    out->push_back(ins);
  }
  int use(int v) const {
    auto it = uses.find(v);
    return it == uses.end() ? 0 : it->second;
  }
  bool is_x(int v) const { return xcls.count(v) != 0; }
  bool live(int r) const { return reg[r] != kEmpty && use(reg[r]) > 0; }
  int where(int v, int avoid = -1) const {
    for (int r = 0; r < 2 + ns; ++r)
      if (r != avoid && reg[r] == v) return r;
    return -1;
  }
  int holders(int v) const {
    int n = 0;
    for (int r : reg)
      if (r == v) ++n;
    return n;
  }
  void count_live() {
    int n = 0;
    for (int r = 2; r < 2 + ns; ++r)
      if (live(r)) ++n;
    max_live = std::max(max_live, n);
  }
  void move(int from, int to) {
    static const int a2s = F_A2S0, b2s = F_B2S0, s2a = F_S02A, s2b = F_S02B;
    int f;
    if (from == RA && to == RB) f = F_A2B;
    else if (from == RB && to == RA) f = F_B2A;
    else if (from == RA) f = a2s + (to - 2);
    else if (from == RB) f = b2s + (to - 2);
    else if (to == RA) f = s2a + (from - 2);
    else f = s2b + (from - 2);
    emit(f);
    reg[to] = reg[from];
  }
  // keep the value in register r alive elsewhere before r is overwritten
  // keep register r's value, if it is still needed, somewhere else before r
  // is overwritten.  to_b: B may take it (not when B holds an operand of
  // the op about to be emitted, whose remaining reads are already counted
  // down)
  void save(int r, bool to_b = true) {
    if (!live(r) || holders(reg[r]) > 1) return;
    // B holds nothing still needed: keep A's value there (a move within
    // the two working registers, no spill slot)
    if (r == RA && to_b && !live(RB)) {
      move(RA, RB);
      return;
    }
    for (int s = 2; s < 2 + ns; ++s)
      if (!live(s)) {
        move(r, s);
        count_live();
        return;
      }
    ok = false;
    why = "op-program needs more than the kernel's spill slots";
  }
  int load_form(int t, int r) const {
    const int base = r == RA ? F_LD_F32_A : F_LD_F32_B;
    switch (p.tensors[t].dtype) {
      case GTF_F32: return base;
      case GTF_BF16: return base + 1;
      default: return base + 2;
    }
  }
  // make register r (A or B) hold v, without disturbing the other of A/B
  void bring(int v, int r) {
    if (reg[r] == v) return;
    save(r);
    const int from = where(v, r);
    if (from >= 0) {
      move(from, r);
    } else if (loadable.count(v)) {
      emit(load_form(v, r), ext_slot.at(v));
      reg[r] = v;
    } else if (is_x(v)) {
      const bool col = xcls.at(v) == CLS_COL;
      emit(r == RA ? (col ? F_COL_A : F_ROW_A) : (col ? F_COL_B : F_ROW_B), lds_slot.at(v));
      reg[r] = v;
    } else {
      ok = false;
      why = "internal: operand not available";
    }
  }
  // A is about to be overwritten by the result of an op that read `a` there
  void consume_a(int a) {
    uses[a] -= 1;
    save(RA);
  }
  void x_info(int v, int* base, int* arg) {
    *base = xcls.at(v) == CLS_COL ? F_ADD_C : F_ADD_R;
    *arg = lds_slot.at(v);
  }

  // A = f(B) or A = B op imm when the operand is (or is best loaded) in B:
  // B keeps a value that is read again, with no move.  False when the
  // operand is better taken in A.
  bool from_b(int v, int form, float imm = 0.f) {
    if (form < 0) return false;
    if (where(v) < 0 && loadable.count(v) && use(v) > 1 && !live(RB)) {
      // read again later: loaded into B, where it stays
      emit(load_form(v, RB), ext_slot.at(v));
      reg[RB] = v;
    }
    if (reg[RB] != v || reg[RA] == v) return false;
    uses[v] -= 1;
    save(RA, false);  // A's value, if still read, goes to a slot: B holds v
    emit(form, 0, imm);
    return true;
  }
  static int b_form(int form) {
    switch (form) {
      case F_EXP: return F_EXP_B;
      case F_TANH: return F_TANH_B;
      case F_RELU: return F_RELU_B;
      case F_SQUARE: return F_SQUARE_B;
      case F_NEG: return F_NEG_B;
    }
    return -1;
  }
  void run_unary(const MOp& m) {
    if (from_b(m.in[0], b_form(m.form))) {
      reg[RA] = m.out;
      return;
    }
    bring(m.in[0], RA);
    consume_a(m.in[0]);
    emit(m.form);
    reg[RA] = m.out;
  }
  void run_copy(const MOp& m) {
    bring(m.in[0], RA);
    consume_a(m.in[0]);
    reg[RA] = m.out;
  }
  // an addressed load into A: the source's slot carries the strides that
  // map a domain position to the source element
  void run_vload(const MOp& m) {
    save(RA);
    if (!ok) return;
    const bool bf = p.tensors[m.src[0]].dtype == GTF_BF16;
    if (m.gkind == 0)
      emit(load_form(m.src[0], RA), ext_slot.at(m.src[0]));
    else if (m.gkind == 3 && ns == 0)  // the tile instance is the wide one without spill slots
      emit(F_LDT_A, 0);
    else if (m.gkind == 1 || m.gkind == 3)
      emit(bf ? F_LDG_BF16_A : F_LDG_F32_A, ext_slot.at(m.src[0]));
    else
      emit(bf ? F_LDC_BF16_A : F_LDC_F32_A, ext_slot.at(m.src[0]) | (ext_slot.at(m.src[1]) << 8),
           m.imm);
    reg[RA] = m.out;
  }
  void run_imm(const MOp& m) {
    if (from_b(m.in[0], F_ADD_IB + m.form, m.imm)) {
      reg[RA] = m.out;
      return;
    }
    bring(m.in[0], RA);
    consume_a(m.in[0]);
    emit(F_ADD_I + m.form, 0, m.imm);
    reg[RA] = m.out;
  }
  void run_binary(const MOp& m) {
    int a = m.in[0], b = m.in[1];
    const bool xa = is_x(a), xb = is_x(b);
    if (xb || (xa && !xb)) {
      // one operand read as X straight from LDS
      const int s = xb ? a : b, x = xb ? b : a;
      if (xa && xb) {
        bring(a, RA);  // a broadcast value pushed into A
        uses[a] -= 0;
      } else {
        bring(s, RA);
        consume_a(s);
      }
      int base, arg;
      x_info(x, &base, &arg);
      emit(base + xop_of(m.form, /*x_on_left=*/!xb), arg);
      reg[RA] = m.out;
      return;
    }
    // both operands are values: A op B, or B (op) A with the reversed form
    int cost_ab = (reg[RA] == a ? 0 : 1) + (reg[RB] == b ? 0 : 1);
    int cost_ba = (reg[RA] == b ? 0 : 1) + (reg[RB] == a ? 0 : 1);
    const bool swap = a != b && cost_ba < cost_ab;
    const int first = swap ? b : a, second = swap ? a : b;
    bring(first, RA);
    if (a == b) {
      save(RB);
      move(RA, RB);
    } else {
      bring(second, RB);
    }
    uses[a] -= 1;
    uses[b] -= 1;
    save(RA, false);  // B keeps its value: the op reads it
    emit(swap ? F_ADD + xop_of(m.form, true) : F_ADD + xop_of(m.form, false));
    reg[RA] = m.out;
  }
  void run_reduce(const MOp& m) {
    bring(m.in[0], RA);
    uses[m.in[0]] -= 1;
    emit(m.form);
  }
};

}  // namespace

// Every index a compiled program hands the executor, checked against what
// the launch provides: external slots, LDS slots, spill slots of the
// instance and the phase each form may appear in.  A failure here is a
// compiler bug, reported before anything is launched.
const char* check_program(const ExecArgs& a, int n_slots) {
  if (a.n_stages < 1 || a.n_stages > kMaxStages) return "stage count out of range";
  if (a.n_col < 0 || a.n_col > kMaxInstr) return "column program out of range";
  if (a.n_col_slots < 0 || a.n_col_slots > kMaxLdsCol) return "column slots out of range";
  if (a.n_row_slots < 0 || a.n_row_slots > kMaxLdsRow) return "row slots out of range";
  if (n_slots < 0 || n_slots > kMaxSlots) return "slot count out of range";
  if (a.RB < 1 || (a.RB % (kBlock >> a.tpr_log2)) != 0) return "row block is not whole passes of the workgroup";
  const int ns = a.NS;
  auto check = [&](int off, int len, int phase) -> const char* {
    // phase 0 column, 1 row, 2 element
    if (off < 0 || len < 0 || off + len > kMaxInstr) return "program out of the buffer";
    for (int i = off; i < off + len; ++i) {
      const int f = a.prog[i].code, arg = a.prog[i].arg;
      if (f < 0 || f >= F_COUNT) return "unknown form";
      if (f <= F_LD_U8_B || f == F_ST_F32 || f == F_ST_BF16) {
        if (arg >= n_slots) return "external slot out of range";
      } else if (f == F_LDG_F32_A || f == F_LDG_BF16_A) {
        if (phase != 2 || arg >= n_slots) return "gather slot out of range";
      } else if (f == F_LDC_F32_A || f == F_LDC_BF16_A) {
        if (phase == 1 || (arg & 0xFF) >= n_slots || (arg >> 8) >= n_slots)
          return "concat slots out of range";
      } else if (f == F_LDT_A) {
        if (phase != 2 || arg >= a.n_tr || a.tr_slot >= n_slots || a.tr_stride < a.PW + 1)
          return "transposed tile out of range";
      } else if (f == F_COL_A || f == F_COL_B || (f >= F_ADD_C && f <= F_MIN_C)) {
        if (phase == 0 || arg >= a.n_col_slots) return "LDS column slot out of range";
      } else if (f == F_ROW_A || f == F_ROW_B || (f >= F_ADD_R && f <= F_MIN_R)) {
        if (phase == 0 || arg >= a.n_row_slots) return "LDS row slot out of range";
      } else if (f == F_ST_LDS) {
        if (phase == 2 || arg >= (phase == 0 ? a.n_col_slots : a.n_row_slots))
          return "LDS store out of range";
      } else if (f == F_RED || f == F_RED_MAX || f == F_RED_MV || f == F_RED_SE) {
        if (phase != 2) return "reduction outside the element phase";
      } else if (f >= F_A2S0 && f <= F_S52B) {
        if ((f - F_A2S0) % kNS >= ns) return "spill slot beyond the instance";
      }
    }
    return nullptr;
  };
  if (const char* e = check(0, a.n_col, 0)) return e;
  for (int st = 0; st < a.n_stages; ++st) {
    const StageDesc& S = a.stage[st];
    if (const char* e = check(S.row_off, S.row_len, 1)) return e;
    if (const char* e = check(S.el_off, S.el_len, 2)) return e;
    if (S.red < 0 || S.red > 5) return "reduction kind out of range";
    if (S.red_lds >= a.n_row_slots || S.red_slot >= n_slots) return "reduction target out of range";
    if (S.red == 0 && (S.red_lds >= 0 || S.red_slot >= 0)) return "reduction target without a reduction";
    if (S.red2_lds >= a.n_row_slots || S.red2_slot >= n_slots) return "reduction target out of range";
    if (S.red < 4 && (S.red2_lds >= 0 || S.red2_slot >= 0)) return "second result without a paired reduction";
  }
  return nullptr;
}

bool compile_group(const FusePlan& p, const std::vector<int>& ops_in, CompiledGroup* outp,
                   std::string* why) {
  CompiledGroup cg;
  std::memset(&cg.args, 0, sizeof(cg.args));
  auto bad = [&](const std::string& s) {
    if (why) *why = s;
    return false;
  };
  // ---- moves folded into a join: a transpose or reshape of a tensor in
  // memory whose value only a concat or a tuple of the group reads (and
  // that is no graph output, in its source's dtype) is that join's
  // addressing of its source, and is not run on its own.  fold: moved value -> (source, (rstride,
  // cstride)), the source's element for position (r, c) of the value.
  std::map<int, std::pair<int, std::pair<int64_t, int64_t>>> fold;
  std::vector<int> ops;
  {
    std::vector<char> in_group(p.ops.size(), 0);
    std::set<int> made;
    for (int i : ops_in) {
      in_group[i] = 1;
      made.insert(p.ops[i].out);
    }
    for (int i : ops_in) {
      const OpInfo& o = p.ops[i];
      if ((o.opcode == GTF_OP_TRANSPOSE || o.opcode == GTF_OP_RESHAPE) && !made.count(o.in[0]) &&
          p.tensors[o.out].role != GTF_ROLE_OUT && p.tensors[o.in[0]].dtype == p.tensors[o.out].dtype) {
        int reader = -1, n = 0;
        for (size_t j = 0; j < p.ops.size(); ++j)
          for (int k = 0; k < p.ops[j].n_in; ++k)
            if (p.ops[j].in[k] == o.out) {
              reader = (int)j;
              ++n;
            }
        if (n == 1 && in_group[reader] && is_join(p.ops[reader])) {
          const int x = o.in[0];
          const TensorInfo& tv = p.tensors[o.out];
          fold[o.out] = {x, o.opcode == GTF_OP_TRANSPOSE
                                ? std::make_pair((int64_t)1, p.tensors[x].C)
                                : std::make_pair(tv.R == 1 ? (int64_t)0 : tv.C, (int64_t)1)};
          continue;
        }
      }
      ops.push_back(i);
    }
  }
  auto source_of = [&](int t) {
    auto f = fold.find(t);
    return f == fold.end() ? t : f->second.first;
  };
  std::vector<char> member(p.ops.size(), 0);
  for (int i : ops) member[i] = 1;
  std::set<int> produced;
  for (int i : ops) produced.insert(p.ops[i].out);

  // ---- addressed loads: a transpose, reshape or concat reads its inputs
  // from memory (none made in the group, none read by another member), so
  // each input's slot carries one mapping from domain positions to its
  // elements
  bool gathers2d = false;
  for (int i : ops) {
    const OpInfo& o = p.ops[i];
    if (!is_gather(o)) continue;
    if (o.opcode != GTF_OP_RESHAPE) gathers2d = true;
    for (int k = 0; k < o.n_in; ++k) {
      if (produced.count(o.in[k])) return bad("transpose/reshape/concat of a value made in the group");
      const int src = source_of(o.in[k]);
      for (int j : ops)
        if (j != i)
          for (int q = 0; q < p.ops[j].n_in; ++q)
            if (p.ops[j].in[q] == o.in[k] || source_of(p.ops[j].in[q]) == src)
              return bad("transpose/reshape/concat input also read by another op of the group");
    }
    if (o.opcode != GTF_OP_RESHAPE && p.tensors[o.in[0]].dtype == GTF_U8)
      return bad("transpose/concat of u8");
  }
  // ---- domain (a gather's input is addressed through it, not broadcast)
  int64_t R = 0, C = 0;
  std::set<int> touched;
  for (int i : ops) {
    const OpInfo& o = p.ops[i];
    if (!is_gather(o))
      for (int k = 0; k < o.n_in; ++k) touched.insert(o.in[k]);
    touched.insert(o.out);
  }
  R = 1;
  C = 1;
  for (int t : touched) {  // extents of 1 broadcast (also to 0)
    if (p.tensors[t].R != 1) R = p.tensors[t].R;
    if (p.tensors[t].C != 1) C = p.tensors[t].C;
  }
  for (int t : touched) {
    const TensorInfo& ti = p.tensors[t];
    if ((ti.R != 1 && ti.R != R) || (ti.C != 1 && ti.C != C)) return bad("shapes in group do not broadcast");
  }
  // ---- reductions
  std::vector<int> reds;
  for (int i : ops)
    if (is_reduce(p.ops[i].opcode)) reds.push_back(i);
  for (int r : reds) {
    const TensorInfo& ri = p.tensors[p.ops[r].in[0]];
    if (ri.R != R || ri.C != C) return bad("reduction input is not the group domain");
  }
  // ---- paired reductions.  In a group that reads its own row results, a
  // mean followed by the mean of squared deviations from it, or a max
  // followed by the sum of exp(x - max), over one input, with nothing else
  // reading the deviations or the squares / exponentials: one pass over the
  // row gives both results (the executor's mean-and-variance and
  // max-and-sum-of-exponentials accumulators), and the two element ops
  // between them are not emitted.
  std::map<int, int> pair_first;  // second reduction -> first
  std::map<int, int> pair_second; // first reduction -> second
  std::set<int> absorbed;         // element ops folded into a paired pass
  {
    std::map<int, int> made_by;
    for (int i : ops) made_by[p.ops[i].out] = i;
    auto n_readers = [&](int t) {
      int n = 0;
      for (const OpInfo& o : p.ops)
        for (int k = 0; k < o.n_in; ++k) n += o.in[k] == t;
      return n;
    };
    for (int r2 : reds) {
      const OpInfo& o2 = p.ops[r2];
      const bool mv = o2.opcode == GTF_OP_ROW_MEAN;
      if (!mv && o2.opcode != GTF_OP_ROW_SUM) continue;
      const int t1 = o2.in[0];
      if (!made_by.count(t1)) continue;
      const int j = made_by[t1];
      if (p.ops[j].opcode != (mv ? GTF_OP_SQUARE : GTF_OP_EXP)) continue;
      const int t2 = p.ops[j].in[0];
      if (!made_by.count(t2)) continue;
      const int k = made_by[t2];
      if (p.ops[k].opcode != GTF_OP_SUB) continue;
      const int x = p.ops[k].in[0], m = p.ops[k].in[1];
      if (!made_by.count(m)) continue;
      const int r1 = made_by[m];
      if (p.ops[r1].opcode != (mv ? GTF_OP_ROW_MEAN : GTF_OP_ROW_MAX) || p.ops[r1].in[0] != x) continue;
      if (n_readers(t1) != 1 || n_readers(t2) != 1) continue;
      if (p.tensors[t1].role == GTF_ROLE_OUT || p.tensors[t2].role == GTF_ROLE_OUT) continue;
      if (pair_second.count(r1) || pair_first.count(r1)) continue;
      pair_first[r2] = r1;
      pair_second[r1] = r2;
      absorbed.insert(j);
      absorbed.insert(k);
    }
  }
  bool flat = reds.empty() && !gathers2d;
  for (int t : touched)
    if (p.tensors[t].R != R || p.tensors[t].C != C) flat = false;
  int64_t DR = flat ? 1 : R, DC = flat ? R * C : C;

  auto cls_of = [&](int t) -> int {
    const TensorInfo& ti = p.tensors[t];
    if (flat) return CLS_E;
    if (ti.R == R && ti.C == C) return CLS_E;
    if (ti.R == 1 && ti.C == C) return CLS_COL;
    return CLS_ROW;
  };
  auto op_cls = [&](int i) -> int {
    if (is_reduce(p.ops[i].opcode)) return CLS_E;
    return cls_of(p.ops[i].out);
  };

  // ---- external slots: inputs read from outside, outputs needed outside
  std::vector<int> slots;
  auto slot_for = [&](int t) {
    for (size_t k = 0; k < slots.size(); ++k)
      if (slots[k] == t) return (int)k;
    slots.push_back(t);
    return (int)slots.size() - 1;
  };
  std::set<int> outputs;
  for (int t : produced) {
    if (p.tensors[t].role == GTF_ROLE_OUT) outputs.insert(t);
    for (size_t j = 0; j < p.ops.size(); ++j) {
      if (member[j]) continue;
      for (int k = 0; k < p.ops[j].n_in; ++k)
        if (p.ops[j].in[k] == t) outputs.insert(t);
    }
  }
  std::set<int> ext_in;
  for (int i : ops)
    for (int k = 0; k < p.ops[i].n_in; ++k)
      if (!produced.count(p.ops[i].in[k])) ext_in.insert(source_of(p.ops[i].in[k]));
  for (int t : ext_in) slot_for(t);
  for (int t : outputs) slot_for(t);
  if ((int)slots.size() > kMaxSlots) return bad("too many external tensors");

  // ---- stages.  A row reduction's result can be read in the group only
  // one stage later: it is known once every element of the row has been
  // added.  Element ops (and reductions) run in the stage of their latest
  // input; row ops in the row program before that stage; column ops in the
  // column phase.  Reading an in-group reduction result is the
  // row-resident extension: the fusion pass keeps a reduction as the last
  // op of its group unless asked to merge across it.
  std::map<int, int> avail;     // produced tensor -> first stage that can read it
  std::map<int, int> stage_of;  // op -> element stage / row program index
  std::map<int, int> producer;  // produced tensor -> op
  for (int i : ops) producer[p.ops[i].out] = i;
  int n_stages = 1;
  for (int i : ops) {
    const OpInfo& o = p.ops[i];
    if (absorbed.count(i)) continue;
    int st = 0;
    if (pair_first.count(i)) {
      st = stage_of.at(pair_first.at(i));  // the first reduction's pass
    } else {
      for (int k = 0; k < o.n_in; ++k)
        if (produced.count(o.in[k])) st = std::max(st, avail.at(o.in[k]));
    }
    const int c = op_cls(i);
    if (c == CLS_COL && st > 0) return bad("column op after a row reduction");
    stage_of[i] = st;
    avail[o.out] = is_reduce(o.opcode) ? st + 1 : st;
    n_stages = std::max(n_stages, st + 1);
  }
  for (int r : reds) {
    bool read_in_group = false;
    for (int i : ops)
      for (int k = 0; k < p.ops[i].n_in; ++k)
        if (p.ops[i].in[k] == p.ops[r].out) read_in_group = true;
    if (read_in_group && cls_of(p.ops[r].out) != CLS_ROW)
      return bad("row reduction over a single column read in its group");
  }
  if (n_stages > kMaxStages) return bad("more row-resident stages than the kernel holds");
  std::vector<int> stage_red(n_stages, -1), stage_red2(n_stages, -1);
  for (int r : reds) {
    if (pair_first.count(r)) {
      stage_red2[stage_of.at(r)] = r;
      continue;
    }
    if (stage_red[stage_of[r]] >= 0) return bad("two row reductions in one stage");
    stage_red[stage_of[r]] = r;
  }

  // ---- operand classes and LDS slots.  ROW/COL values read by element
  // ops live in LDS; so do row values that cross from one row program (or
  // a reduction) to a later row program.
  std::map<int, int> row_lds, col_lds;
  auto need_row = [&](int t) {
    if (!row_lds.count(t)) {
      const int s = (int)row_lds.size();
      row_lds[t] = s;
    }
  };
  for (int i : ops) {
    const OpInfo& o = p.ops[i];
    if (is_gather(o) || absorbed.count(i)) continue;  // loaded addressed / not emitted
    const int c = op_cls(i);
    for (int k = 0; k < o.n_in; ++k) {
      const int t = o.in[k];
      const int ci = cls_of(t);
      if (c == CLS_E) {
        if (ci == CLS_ROW) need_row(t);
        if (ci == CLS_COL && !col_lds.count(t)) {
          const int s = (int)col_lds.size();
          col_lds[t] = s;
        }
      } else if (c == CLS_ROW && produced.count(t)) {
        const int j = producer.at(t);
        if (is_reduce(p.ops[j].opcode) || stage_of.at(j) != stage_of.at(i)) need_row(t);
      }
    }
  }
  if ((int)row_lds.size() > kMaxLdsRow) return bad("too many row operands");
  if ((int)col_lds.size() > kMaxLdsCol) return bad("too many column operands");
  // row / column ops may read only their own class (column ops may also
  // load an external [1,1] scalar)
  for (int i : ops) {
    int c = op_cls(i);
    if (c == CLS_E || is_gather(p.ops[i])) continue;
    const OpInfo& o = p.ops[i];
    for (int k = 0; k < o.n_in; ++k) {
      int ci = cls_of(o.in[k]);
      if (ci == c) continue;
      bool ext_scalar = !produced.count(o.in[k]) && p.tensors[o.in[k]].R == 1 &&
                        p.tensors[o.in[k]].C == 1;
      if (c == CLS_COL && ext_scalar) continue;
      return bad("row/column operand mix not supported in one group");
    }
  }

  // ---- sums reduced term by term.  A row sum or mean whose input is an
  // add or add3 made in the group, read by nothing else and not stored, over
  // full-domain values, adds each of its terms into the row accumulator
  // instead: the sum of the terms' sums is the sum (only the order of the
  // roundings moves, well inside the reduction tolerance), the adds are not
  // run, and the group holds one value fewer at a time.  Nested adds expand
  // the same way.
  std::map<int, std::vector<int>> red_terms;  // reduction op -> the tensors it sums
  {
    std::map<int, int> n_read;
    for (const OpInfo& o : p.ops)
      for (int k = 0; k < o.n_in; ++k) n_read[o.in[k]] += 1;
    std::set<int> summed;
    std::function<void(int, std::vector<int>&, std::vector<int>&)> expand =
        [&](int t, std::vector<int>& terms, std::vector<int>& adds) {
          auto it = producer.find(t);
          bool open = it != producer.end() && !absorbed.count(it->second) &&
                      (p.ops[it->second].opcode == GTF_OP_ADD || p.ops[it->second].opcode == GTF_OP_ADD3) &&
                      n_read[t] == 1 && !outputs.count(t) && cls_of(t) == CLS_E;
          if (open)
            for (int k = 0; k < p.ops[it->second].n_in; ++k)
              if (cls_of(p.ops[it->second].in[k]) != CLS_E) open = false;
          if (!open) {
            terms.push_back(t);
            return;
          }
          adds.push_back(it->second);
          for (int k = 0; k < p.ops[it->second].n_in; ++k) expand(p.ops[it->second].in[k], terms, adds);
        };
    for (int r : reds) {
      const OpInfo& o = p.ops[r];
      if (o.opcode != GTF_OP_ROW_SUM && o.opcode != GTF_OP_ROW_MEAN) continue;
      if (pair_first.count(r) || pair_second.count(r)) continue;
      std::vector<int> terms, adds;
      expand(o.in[0], terms, adds);
      if (adds.empty()) continue;
      red_terms[r] = terms;
      for (int j : adds) summed.insert(j);
    }
  }

  // ---- lower each op to micro-ops
  std::map<int, std::vector<MOp>> mops_of;
  std::map<int, std::pair<int64_t, int64_t>> gather_stride;  // source tensor -> (rstride, cstride)
  int n_tr = 0, tr_src = -1;  // the transposed source staged in LDS
  int synth = -1;
  for (int i : ops) {
    const OpInfo& o = p.ops[i];
    auto& L = mops_of[i];
    if (is_gather(o)) {
      // the source's element for domain position (r, c), by the op's own
      // index map; a plain load when that map is the value's own layout
      MOp m;
      m.kind = 5;
      m.out = o.out;
      m.src[0] = o.in[0];
      const TensorInfo& to = p.tensors[o.out];
      const int ct = cls_of(o.out);
      auto own = [&](int64_t Rt, int64_t Ct) -> std::pair<int64_t, int64_t> {
        if (flat) return {0, 1};
        if (ct == CLS_E) return {Ct, 1};
        if (ct == CLS_COL) return {0, 1};
        return {Rt == 1 ? 0 : 1, 0};
      };
      if (is_join(o)) {
        if (ct == CLS_ROW) return bad("concat of per-row values");
        const TensorInfo& a = p.tensors[o.in[0]];
        // each side from memory at its own layout, or through a folded move
        auto side = [&](int t) -> std::pair<int, std::pair<int64_t, int64_t>> {
          auto f = fold.find(t);
          if (f != fold.end()) return f->second;
          const TensorInfo& ti = p.tensors[t];
          return {t, {ti.R == 1 ? 0 : ti.C, 1}};
        };
        const auto sa = side(o.in[0]), sb = side(o.in[1]);
        if (sa.first == sb.first && sa.second != sb.second) return bad("one tensor read at two layouts");
        m.gkind = 2;
        m.src[0] = sa.first;
        m.src[1] = sb.first;
        m.imm = (float)a.C;
        if (a.C > (1 << 24)) return bad("concat split column beyond fp32 integers");
        gather_stride[sa.first] = sa.second;
        gather_stride[sb.first] = sb.second;
      } else if (o.opcode == GTF_OP_TRANSPOSE && ct == CLS_E) {
        // T[r][c] = X[c][r]: X is [C, R] in domain terms.  One such source
        // of a group without reductions is staged per item in LDS, read in
        // coalesced X rows (tiled); others are read element by element
        gather_stride[o.in[0]] = {1, p.tensors[o.in[0]].C};
        if (reds.empty() && n_tr == 0) {
          m.gkind = 3;
          n_tr = 1;
          tr_src = o.in[0];
        } else {
          m.gkind = 1;
        }
      } else {
        // reshape (row-major order kept), or a transpose of a vector, is
        // the result's own layout over the source's memory
        m.gkind = 0;
        gather_stride[o.in[0]] = own(to.R, to.C);
      }
      L.push_back(m);
      continue;
    }
    if (o.opcode == GTF_OP_COPY || o.opcode == GTF_OP_CONCAT) {  // (a concat of one tuple)
      MOp m;
      m.kind = 4;
      m.form = 0;
      m.in[0] = o.in[0];
      m.out = o.out;
      L.push_back(m);
    } else if (unary_form(o.opcode) >= 0) {
      MOp m;
      m.kind = 0;
      m.form = unary_form(o.opcode);
      m.in[0] = o.in[0];
      m.out = o.out;
      L.push_back(m);
    } else if (o.opcode == GTF_OP_ADD_IMM || o.opcode == GTF_OP_MUL_IMM) {
      MOp m;
      m.kind = 2;
      m.form = o.opcode == GTF_OP_ADD_IMM ? X_ADD : X_MUL;
      m.imm = o.imm;
      m.in[0] = o.in[0];
      m.out = o.out;
      L.push_back(m);
    } else if (binary_form(o.opcode) >= 0) {
      MOp m;
      m.kind = 1;
      m.form = binary_form(o.opcode);
      m.commutative = commutative(m.form);
      m.in[0] = o.in[0];
      m.in[1] = o.in[1];
      m.out = o.out;
      L.push_back(m);
    } else if (o.opcode == GTF_OP_ADD3) {
      MOp m1;
      m1.kind = 1;
      m1.form = F_ADD;
      m1.commutative = true;
      m1.in[0] = o.in[0];
      m1.in[1] = o.in[1];
      m1.out = --synth;
      MOp m2 = m1;
      m2.in[0] = m1.out;
      m2.in[1] = o.in[2];
      m2.out = o.out;
      L.push_back(m1);
      L.push_back(m2);
    } else if (o.opcode == GTF_OP_DMUL) {
      MOp m1;
      m1.kind = 2;
      m1.form = X_MUL;
      m1.imm = o.imm;
      m1.in[0] = o.in[0];
      m1.out = --synth;
      MOp m2;
      m2.kind = 1;
      m2.form = F_MUL;
      m2.commutative = true;
      m2.in[0] = m1.out;
      m2.in[1] = o.in[1];
      m2.out = o.out;
      L.push_back(m1);
      L.push_back(m2);
    } else if (is_reduce(o.opcode)) {
      MOp m;
      m.kind = 3;
      m.form = o.opcode == GTF_OP_ROW_MAX ? F_RED_MAX : F_RED;
      if (pair_second.count(i)) m.form = o.opcode == GTF_OP_ROW_MEAN ? F_RED_MV : F_RED_SE;
      m.in[0] = o.in[0];
      m.out = o.out;
      if (red_terms.count(i)) {
        for (int t : red_terms.at(i)) {  // one accumulation per term
          m.in[0] = t;
          L.push_back(m);
        }
      } else {
        L.push_back(m);
      }
    } else {
      return bad("unsupported opcode in group");
    }
  }

  // ---- programs: the column program, then per stage a row program and an
  // element program.  A stage's element program is the cone of element ops
  // its sinks need (its reduction, and the outputs first available in it),
  // recomputed from reloaded inputs rather than carried between stages.
  enum PKind { P_COL = 0, P_ROW = 1, P_EL = 2 };
  struct Prog {
    int kind, stage;
    std::vector<MOp> L;
    std::set<int> store;  // values this program stores to their external slots
  };
  std::vector<Prog> progs;
  {
    Prog pc{P_COL, 0, {}, {}};
    for (int i : ops)
      if (op_cls(i) == CLS_COL) {
        for (auto& m : mops_of[i]) pc.L.push_back(m);
        if (outputs.count(p.ops[i].out)) pc.store.insert(p.ops[i].out);
      }
    progs.push_back(pc);
  }
  for (int st = 0; st < n_stages; ++st) {
    Prog pr{P_ROW, st, {}, {}};
    for (int i : ops)
      if (op_cls(i) == CLS_ROW && stage_of[i] == st) {
        for (auto& m : mops_of[i]) pr.L.push_back(m);
        if (outputs.count(p.ops[i].out)) pr.store.insert(p.ops[i].out);
      }
    progs.push_back(pr);
    Prog pe{P_EL, st, {}, {}};
    std::set<int> cone;
    std::vector<int> work;
    if (stage_red[st] >= 0) work.push_back(stage_red[st]);
    for (int i : ops)
      if (op_cls(i) == CLS_E && !is_reduce(p.ops[i].opcode) && !absorbed.count(i) && stage_of.at(i) == st &&
          outputs.count(p.ops[i].out)) {
        work.push_back(i);
        pe.store.insert(p.ops[i].out);
      }
    while (!work.empty()) {
      const int i = work.back();
      work.pop_back();
      if (cone.count(i)) continue;
      cone.insert(i);
      // a reduction summed term by term reads its terms, not the adds
      const std::vector<int> ins = red_terms.count(i)
                                       ? red_terms.at(i)
                                       : std::vector<int>(p.ops[i].in, p.ops[i].in + p.ops[i].n_in);
      for (int t : ins) {
        if (!produced.count(t)) continue;
        const int j = producer.at(t);
        if (op_cls(j) == CLS_E && !is_reduce(p.ops[j].opcode)) work.push_back(j);
      }
    }
    for (int i : ops)
      if (cone.count(i))
        for (auto& m : mops_of[i]) pe.L.push_back(m);
    progs.push_back(pe);
  }
  // A GELU whose value is only rounded to bf16 and stored (no op of the
  // plan reads the tensor) takes the cheaper form, accurate to far below
  // bf16's half ulp
  {
    std::set<int> read;
    for (const auto& o : p.ops)
      for (int k = 0; k < o.n_in; ++k) read.insert(o.in[k]);
    for (auto& P : progs) {
      if (P.kind != P_EL) continue;
      for (auto& m : P.L)
        if (m.kind == 0 && m.form == F_GELU && m.out >= 0 && P.store.count(m.out) &&
            !read.count(m.out) && p.tensors[m.out].dtype == GTF_BF16)
          m.form = F_GELU_BF;
    }
  }

  // ---- code generation, program by program; first for the wide instance
  // without spill slots, then with two, else for the narrow one
  std::vector<std::vector<Instr>> code(progs.size());
  int max_depth = 0;
  auto generate = [&](int ns, bool hoist, std::string* gwhy) -> bool {
    for (auto& c : code) c.clear();
    max_depth = 0;
    for (size_t pi = 0; pi < progs.size(); ++pi) {
      const Prog& P = progs[pi];
      const int ph = P.kind == P_COL ? CLS_COL : P.kind == P_ROW ? CLS_ROW : CLS_E;
      Codegen g{p, &code[pi], ph};
      g.init();
      g.ns = ns;
      for (size_t k = 0; k < slots.size(); ++k) g.ext_slot[slots[k]] = (int)k;
      const auto& L = P.L;
      std::set<int> made_here;
      for (auto& m : L) made_here.insert(m.out);
      // values read from LDS: in element programs every row / column
      // operand; in row programs the row values made elsewhere
      if (P.kind == P_EL) {
        for (auto& kv : row_lds) {
          g.xcls[kv.first] = CLS_ROW;
          g.lds_slot[kv.first] = kv.second;
        }
        for (auto& kv : col_lds) {
          g.xcls[kv.first] = CLS_COL;
          g.lds_slot[kv.first] = kv.second;
        }
      } else if (P.kind == P_ROW) {
        for (auto& kv : row_lds)
          if (produced.count(kv.first) && !made_here.count(kv.first)) {
            g.xcls[kv.first] = CLS_ROW;
            g.lds_slot[kv.first] = kv.second;
          }
      }
      for (auto& m : L) {
        const int n_in = mop_arity(m);
        for (int k = 0; k < n_in; ++k) {
          const int v = m.in[k];
          if (g.is_x(v)) continue;
          g.uses[v] += 1;
          if (v >= 0 && !produced.count(v)) g.loadable.insert(v);
        }
      }
      // externals staged into LDS for the element programs: column operands
      // in the column program, row operands in the first row program
      std::vector<std::pair<int, int>> staging;
      if (P.kind == P_COL)
        for (auto& kv : col_lds)
          if (!produced.count(kv.first)) staging.push_back(kv);
      if (P.kind == P_ROW && P.stage == 0)
        for (auto& kv : row_lds)
          if (!produced.count(kv.first)) staging.push_back(kv);
      for (auto& kv : staging) g.loadable.insert(kv.first);
      // load hoisting: the program's first two external loads (in order of
      // first use) go to A and B at once, so both are in flight together
      if (hoist) {
        std::vector<int> first_use;
        auto note = [&](int v) {
          if (g.loadable.count(v) && std::find(first_use.begin(), first_use.end(), v) == first_use.end())
            first_use.push_back(v);
        };
        for (auto& kv : staging) note(kv.first);
        for (auto& m : L)
          for (int k = 0; k < mop_arity(m); ++k) note(m.in[k]);
        // (a lone input read more than once goes to B, where the unary and
        // immediate forms read it without moving it)
        const bool lone_in_b = first_use.size() == 1 && g.use(first_use[0]) > 1;
        for (size_t i = 0; i < first_use.size() && i < 2; ++i) {
          const int r = i == 0 && !lone_in_b ? Codegen::RA : Codegen::RB;
          g.emit(g.load_form(first_use[i], r), g.ext_slot.at(first_use[i]));
          g.reg[r] = first_use[i];
        }
      }
      for (auto& kv : staging) {
        g.bring(kv.first, Codegen::RA);
        g.emit(F_ST_LDS, kv.second);
      }
      // list scheduling: among ready micro-ops prefer one whose operands
      // already sit in A (and B)
      std::vector<char> done(L.size(), 0);
      std::set<int> ready_vals;
      for (size_t step = 0; step < L.size() && g.ok; ++step) {
        int best = -1, best_score = -1;
        for (size_t k = 0; k < L.size(); ++k) {
          if (done[k]) continue;
          const int n_in = mop_arity(L[k]);
          bool rdy = true;
          for (int q = 0; q < n_in; ++q)
            if (made_here.count(L[k].in[q]) && !ready_vals.count(L[k].in[q])) rdy = false;
          if (!rdy) continue;
          // every binary op has a reversed form, so either operand may sit in A
          const int x0 = L[k].in[0], x1 = n_in == 2 ? L[k].in[1] : kNoValue;
          const int ra = g.reg[Codegen::RA], rb = g.reg[Codegen::RB];
          int score = 0;
          if (ra == x0 || ra == x1) score += 2;
          if (n_in == 2 && ((rb == x1 && ra != x1) || (rb == x0 && ra != x0))) score += 1;
          // a unary or immediate op reads its operand from B too (after ops
          // that free A by reading it)
          if (n_in == 1 && rb == x0 && ra != x0 &&
              (L[k].kind == 2 || (L[k].kind == 0 && Codegen::b_form(L[k].form) >= 0)))
            score += 1;
          if (score > best_score) {
            best_score = score;
            best = (int)k;
          }
        }
        if (best < 0) {
          *gwhy = "internal: no ready op";
          return false;
        }
        done[best] = 1;
        const MOp& m = L[best];
        switch (m.kind) {
          case 0: g.run_unary(m); break;
          case 1: g.run_binary(m); break;
          case 2: g.run_imm(m); break;
          case 3: g.run_reduce(m); break;
          case 5: g.run_vload(m); break;
          default: g.run_copy(m); break;
        }
        if (!g.ok) break;
        if (m.kind == 3) continue;
        ready_vals.insert(m.out);
        const int v = m.out;
        if (v >= 0 && P.store.count(v))
          g.emit(p.tensors[v].dtype == GTF_BF16 ? F_ST_BF16 : F_ST_F32, g.ext_slot.at(v));
        if (P.kind == P_COL && v >= 0 && col_lds.count(v)) g.emit(F_ST_LDS, col_lds.at(v));
        if (P.kind == P_ROW && v >= 0 && row_lds.count(v)) g.emit(F_ST_LDS, row_lds.at(v));
      }
      if (!g.ok) {
        *gwhy = g.why;
        return false;
      }
      max_depth = std::max(max_depth, g.max_live);
    }
    return true;
  };
  // instances in order of preference: wide with no spill slot (highest
  // occupancy), wide with two, narrow with six
  int ns = -1;
  {
    std::string w;
    const int tries[3] = {0, kWideNS, kNS};
    for (int n : tries) {
      if (generate(n, true, &w) || generate(n, false, &w)) {
        ns = n;
        break;
      }
    }
    if (ns < 0) return bad(w);
  }
  if (ns != 0) n_tr = 0;  // the transposed source is read element by element instead
  const int K = ns == kNS ? 1 : kWideK;

  size_t total = 0;
  for (auto& c : code) total += c.size();
  if (total > (size_t)kMaxInstr) return bad("op-program longer than the instruction buffer");

  // ---- geometry
  // Work items are (row block, column panel).  A panel is staged in LDS
  // when the group has column operands; a flat group (no broadcast, no
  // reduction) is one row of numel elements cut into panels of one lane
  // tile per thread.  Threads split into rows of tpr lanes; tpr is the
  // largest power of two that still gives each lane K sub-tiles of the row
  // (at most 64 for a reduction over many rows, so each row sums inside one
  // wave).
  ExecArgs& a = cg.args;
  a.R = DR;
  a.C = DC;
  a.K = K;
  a.NS = ns;
  const int64_t C8 = (DC + kV - 1) / kV * kV;
  int pw;
  if (!reds.empty()) {
    pw = (int)std::max<int64_t>(C8, kV);
    if (!col_lds.empty() && (int64_t)col_lds.size() * C8 > 16384)
      return bad("reduction group with column operands wider than the LDS panel");
    if (C8 > (int64_t)1 << 30) return bad("row too wide");
  } else if (flat) {
    pw = kBlock * kV * std::max(K, 2);
  } else if (n_tr > 0) {
    pw = (int)std::min<int64_t>(std::max<int64_t>(C8, kV), 128);  // 64-row by 128-column tiles
  } else {
    pw = (int)std::min<int64_t>(std::max<int64_t>(C8, kV), kPanelMax);
  }
  int64_t n_panels = DC == 0 ? 1 : (DC + pw - 1) / pw;
  const int64_t nt = (pw + kV - 1) / kV;
  int tpr = 1;
  {
    const int64_t want = std::max<int64_t>(1, nt / K);
    while ((int64_t)tpr * 2 <= want && tpr * 2 <= kBlock) tpr <<= 1;
    if (!reds.empty() && tpr > 64 && DR >= 256) tpr = 64;
  }
  // a staged transposed tile is 64 rows (4 lanes per row) by at most 128
  // columns: at most 64 x 129 floats of LDS
  if (n_tr > 0) tpr = 4;
  const int rpp = kBlock / tpr;
  // A row block is one pass of the workgroup's rows, or two passes when
  // that still leaves at least 1024 items (one per resident workgroup of the
  // wide instance on MI355X): each item then walks two runs per lane and
  // its setup (scalar loads, the block's coordinates, the stage's phases)
  // is shared by both.  Measured: bias+GELU [8192,4096] and the row-resident
  // softmax [131072,128] 6% faster, the diamond row sum over bf16[8192,4096]
  // 3.5% faster, relu(X + bias) + R over bf16[4096,4096] 2.5% slower; the
  // LayerNorm groups over [8192,1024], left with 512 items, would be 13-15%
  // slower.
  const int64_t items1 = DR == 0 ? 0 : (DR + rpp - 1) / rpp * n_panels;
  const int rb = n_tr == 0 && !flat && items1 >= 2048 ? 2 * rpp : rpp;
  const int64_t n_rb = DR == 0 ? 0 : (DR + rb - 1) / rb;
  a.n_items = n_rb * n_panels;
  a.n_panels = (int)n_panels;
  a.RB = rb;
  a.PW = pw;
  int lg = 0;
  while ((1 << lg) < tpr) ++lg;
  a.tpr_log2 = lg;
  a.n_col_slots = (int)col_lds.size();
  a.n_row_slots = (int)row_lds.size();
  // program layout: column program, then per stage row and element programs
  size_t pos = 0;
  a.n_col = (int)code[0].size();
  for (const Instr& ins : code[0]) a.prog[pos++] = ins;
  a.n_stages = n_stages;
  for (int st = 0; st < n_stages; ++st) {
    StageDesc& S = a.stage[st];
    const auto& cr = code[1 + 2 * st];
    const auto& ce = code[2 + 2 * st];
    S.row_off = (int)pos;
    S.row_len = (int)cr.size();
    for (const Instr& ins : cr) a.prog[pos++] = ins;
    S.el_off = (int)pos;
    S.el_len = (int)ce.size();
    for (const Instr& ins : ce) a.prog[pos++] = ins;
    S.red = 0;
    S.red_lds = -1;
    S.red_slot = -1;
    S.red_dtype = DT_F32;
    S.red2_lds = -1;
    S.red2_slot = -1;
    S.red2_dtype = DT_F32;
    S.red2_pad_ = 0;
    const int r = stage_red[st];
    if (r >= 0) {
      const int t = p.ops[r].out;
      S.red = p.ops[r].opcode == GTF_OP_ROW_MEAN ? 2 : p.ops[r].opcode == GTF_OP_ROW_MAX ? 3 : 1;
      if (row_lds.count(t)) S.red_lds = row_lds.at(t);
      if (outputs.count(t)) S.red_slot = slot_for(t);
      S.red_dtype = p.tensors[t].dtype == GTF_BF16 ? DT_BF16 : DT_F32;
      const int r2 = stage_red2[st];
      if (r2 >= 0) {
        const int t2 = p.ops[r2].out;
        S.red = S.red == 2 ? 4 : 5;
        if (row_lds.count(t2)) S.red2_lds = row_lds.at(t2);
        if (outputs.count(t2)) S.red2_slot = slot_for(t2);
        S.red2_dtype = p.tensors[t2].dtype == GTF_BF16 ? DT_BF16 : DT_F32;
      }
    }
  }
  for (size_t s = 0; s < slots.size(); ++s) {
    const TensorInfo& ti = p.tensors[slots[s]];
    int c = cls_of(slots[s]);
    auto gs = gather_stride.find(slots[s]);
    if (gs != gather_stride.end()) {
      a.rstride[s] = gs->second.first;
      a.cstride[s] = gs->second.second;
    } else if (flat) {
      a.rstride[s] = 0;
      a.cstride[s] = 1;
    } else if (c == CLS_E) {
      a.rstride[s] = C;
      a.cstride[s] = 1;
    } else if (c == CLS_COL) {
      a.rstride[s] = 0;
      a.cstride[s] = 1;
    } else {
      a.rstride[s] = ti.R == 1 ? 0 : 1;
      a.cstride[s] = 0;
    }
  }
  cg.slot_tensor = slots;
  for (int t : slots) cg.slot_numel.push_back(p.tensors[t].R * p.tensors[t].C);
  for (int t : slots) cg.slot_dtype.push_back(p.tensors[t].dtype);
  cg.n_slots = (int)slots.size();
  cg.max_depth = max_depth;
  a.n_tr = n_tr;
  a.tr_slot = n_tr > 0 ? slot_for(tr_src) : 0;
  a.tr_bf16 = n_tr > 0 && p.tensors[tr_src].dtype == GTF_BF16;
  {
    // a tile row spans every column a lane of a run may read, partial runs
    // included (K sub-tiles of kV, tpr * kV apart), plus one float so that
    // a wave's column writes fall in different banks
    const int64_t ks_ = (int64_t)tpr * kV;
    const int64_t span = ((pw + ks_ - 1) / ks_ + K - 1) / K * K * ks_;
    a.tr_stride = (int)std::max<int64_t>(span, pw) + 1;
  }
  a.tr_off = a.n_col_slots * pw + a.n_row_slots * rb + 16;
  cg.lds_bytes = (int)(a.n_col_slots * (int64_t)pw * 4 + a.n_row_slots * (int64_t)rb * 4 + 16 * 4 +
                       (int64_t)n_tr * rb * a.tr_stride * 4);
  if (cg.lds_bytes > 64 * 1024) return bad("LDS staging exceeds 64 KiB");
  a.slow_only = 0;
  for (size_t k = 0; k < pos; ++k) {
    const int f = a.prog[k].code;
    if (f == F_LDG_F32_A || f == F_LDG_BF16_A || f == F_LDC_F32_A || f == F_LDC_BF16_A) a.slow_only = 1;
  }
  if (const char* why = check_program(a, cg.n_slots)) return bad(why);
  if (outp) *outp = cg;
  return true;
}

// ================================================================ planning
namespace {

// OpPatternKind per op ("Operator Pattern Classification") and the
// post-dominator tree ("Algorithm" step 2).
void annotate(FusePlan* p) {
  for (OpInfo& o : p->ops) {
    if (o.flags & GTF_OPF_OPAQUE) {
      o.pattern = GTF_PAT_OPAQUE;
    } else if (is_reduce(o.opcode)) {
      o.pattern = GTF_PAT_COMM_REDUCE;
    } else if (o.opcode == GTF_OP_TUPLE) {
      o.pattern = GTF_PAT_TUPLE;
    } else if (o.opcode == GTF_OP_COPY || o.opcode == GTF_OP_CONCAT || is_gather(o)) {
      o.pattern = GTF_PAT_INJECTIVE;
    } else {
      const TensorInfo& to = p->tensors[o.out];
      o.pattern = GTF_PAT_ELEMWISE;
      for (int k = 0; k < o.n_in; ++k) {
        const TensorInfo& ti = p->tensors[o.in[k]];
        if (ti.R != to.R || ti.C != to.C) o.pattern = GTF_PAT_BROADCAST;
      }
    }
  }
  auto rd = readers_of(*p);
  p->ipdom = postdom_tree(*p, rd);
}

// The grouping ("Algorithm" step 3, "Fusion rules"), then the optional
// row-resident merge.  Groups are member lists, each ascending, listed in
// the order of their union-find roots.
std::vector<std::vector<int>> partition_groups(const FusePlan& pl, bool fuse, bool row_resident) {
  const FusePlan* p = &pl;
  const int n = (int)p->ops.size();
  auto rd = readers_of(*p);
  std::vector<int> pats(n);
  for (int i = 0; i < n; ++i) pats[i] = p->ops[i].pattern;
  UnionFind uf(pats);
  if (fuse) {
    std::vector<char> mark(n, 0), in_set(n, 0);
    for (int phase = 0; phase < 3; ++phase) {
      for (int i = 0; i < n; ++i) {
        int d = p->ipdom[i];
        if (d < 0 || uf.find(i) == uf.find(d)) continue;
        int src = uf.pat[uf.find(i)];
        int sink = uf.pat[uf.find(d)];
        // CheckPath: ops strictly between i and d on any path
        std::vector<int> between, stack(rd[i].begin(), rd[i].end());
        std::fill(mark.begin(), mark.end(), 0);
        bool path_ok = true;
        while (!stack.empty()) {
          int v = stack.back();
          stack.pop_back();
          if (v == d || mark[v]) continue;
          mark[v] = 1;
          between.push_back(v);
          if (p->ops[v].pattern > GTF_PAT_INJECTIVE) path_ok = false;
          for (int s : rd[v]) stack.push_back(s);
        }
        bool ok;
        if (p->ops[d].opcode == GTF_OP_TUPLE)  // phase 2: fields into a tuple already fused onward
          ok = phase == 2 && src <= GTF_PAT_INJECTIVE && uf.find(d) != d && path_ok;
        else if (src <= GTF_PAT_BROADCAST)
          ok = path_ok && sink <= GTF_PAT_COMM_REDUCE;
        else if ((src == GTF_PAT_INJECTIVE || src == GTF_PAT_TUPLE) && phase >= 1)
          ok = path_ok && sink <= GTF_PAT_INJECTIVE;
        else
          ok = false;
        if (!ok) continue;
        // members of the merged group
        std::set<int> roots{uf.find(i), uf.find(d)};
        for (int v : between) roots.insert(uf.find(v));
        std::fill(in_set.begin(), in_set.end(), 0);
        std::vector<int> members;
        for (int v = 0; v < n; ++v)
          if (roots.count(uf.find(v))) {
            in_set[v] = 1;
            members.push_back(v);
          }
        if ((int)members.size() > GTF_MAX_GROUP_OPS) continue;
        if (count_args(*p, in_set) > GTF_MAX_GROUP_ARGS) continue;
        if (!compile_group(*p, members, nullptr, nullptr)) continue;  // resources
        // CommitFuse
        uf.merge_into(i, d);
        for (int v : between) uf.merge_into(v, d);
      }
    }
  }
  // Row-resident extension (opt-in): a group that ends in a row reduction
  // is merged with a group on the same [R,C] domain that reads the
  // reduction's [R,1] result, so the result never leaves the kernel (a
  // one-kernel LayerNorm).  The merge must keep the group graph acyclic
  // (no op outside the two groups on a path from one to the other) and the
  // op and argument limits, and the kernel must hold the stages it makes.
  if (fuse && row_resident) {
    std::vector<char> in_set(n, 0);
    bool changed = true;
    while (changed) {
      changed = false;
      for (int r = 0; r < n && !changed; ++r) {
        if (!is_reduce(p->ops[r].opcode)) continue;
        const int t = p->ops[r].out;
        for (int c = 0; c < n && !changed; ++c) {
          bool reads = false;
          for (int k = 0; k < p->ops[c].n_in; ++k)
            if (p->ops[c].in[k] == t) reads = true;
          if (!reads || uf.find(c) == uf.find(r)) continue;
          if (p->ops[c].pattern == GTF_PAT_OPAQUE) continue;
          const int gr = uf.find(r), gc = uf.find(c);
          std::fill(in_set.begin(), in_set.end(), 0);
          std::vector<int> members;
          for (int v = 0; v < n; ++v)
            if (uf.find(v) == gr || uf.find(v) == gc) {
              in_set[v] = 1;
              members.push_back(v);
            }
          // convexity: walk forward from the members through non-members; a
          // walk that re-enters the set would become a cycle
          std::vector<char> seen(n, 0);
          std::vector<int> stack;
          for (int v : members)
            for (int w : rd[v])
              if (!in_set[w]) stack.push_back(w);
          bool convex = true;
          while (!stack.empty() && convex) {
            const int v = stack.back();
            stack.pop_back();
            if (seen[v]) continue;
            seen[v] = 1;
            for (int w : rd[v]) {
              if (in_set[w]) convex = false;
              else stack.push_back(w);
            }
          }
          if (!convex) continue;
          if ((int)members.size() > GTF_MAX_GROUP_OPS) continue;
          if (count_args(*p, in_set) > GTF_MAX_GROUP_ARGS) continue;
          if (!compile_group(*p, members, nullptr, nullptr)) continue;
          uf.merge_into(r, c);
          changed = true;
        }
      }
    }
  }
  std::map<int, std::vector<int>> byroot;
  for (int i = 0; i < n; ++i) byroot[uf.find(i)].push_back(i);
  std::vector<std::vector<int>> gl;
  for (auto& kv : byroot) gl.push_back(kv.second);
  return gl;
}

int64_t tensor_bytes(const TensorInfo& t) {
  return t.R * t.C * (t.dtype == GTF_F32 ? 4 : t.dtype == GTF_BF16 ? 2 : 1);
}

// Cost of a grouping: HBM bytes (every distinct tensor a group reads from
// memory, every tensor it stores) and launches.
std::pair<int64_t, int64_t> plan_cost(const FusePlan& p, const std::vector<std::vector<int>>& gl) {
  std::vector<int> owner(p.tensors.size(), -1);
  for (size_t g = 0; g < gl.size(); ++g)
    for (int i : gl[g]) owner[p.ops[i].out] = (int)g;
  std::vector<char> stored(p.tensors.size(), 0);
  for (size_t t = 0; t < p.tensors.size(); ++t)
    if (p.tensors[t].role == GTF_ROLE_OUT) stored[t] = 1;
  for (size_t g = 0; g < gl.size(); ++g)
    for (int i : gl[g])
      for (int k = 0; k < p.ops[i].n_in; ++k) {
        const int t = p.ops[i].in[k];
        if (owner[t] >= 0 && owner[t] != (int)g) stored[t] = 1;
      }
  int64_t bytes = 0;
  for (size_t g = 0; g < gl.size(); ++g) {
    std::set<int> touched;
    for (int i : gl[g]) {
      for (int k = 0; k < p.ops[i].n_in; ++k) {
        const int t = p.ops[i].in[k];
        if (owner[t] != (int)g) touched.insert(t);
      }
      if (stored[p.ops[i].out]) touched.insert(p.ops[i].out);
    }
    for (int t : touched) bytes += tensor_bytes(p.tensors[t]);
  }
  return {bytes, (int64_t)gl.size()};
}

// Duplicate op v for each reader in `targets`: a copy of v, writing a new
// internal tensor, goes right before its reader, which then reads the copy.
// v itself goes when it is an intermediate left without readers.  Returns
// the copies' op ids in the new program.
std::vector<int> duplicate_op(FusePlan* p, int v, const std::vector<int>& targets) {
  const int n = (int)p->ops.size();
  const int tv = p->ops[v].out;
  std::vector<char> is_target(n, 0);
  for (int r : targets) is_target[r] = 1;
  std::vector<int> new_t(n, -1);
  for (int r : targets) {
    TensorInfo ti = p->tensors[tv];
    ti.role = GTF_ROLE_TMP;
    p->tensors.push_back(ti);
    new_t[r] = (int)p->tensors.size() - 1;
  }
  bool v_read = false;
  for (int j = 0; j < n; ++j)
    if (!is_target[j])
      for (int k = 0; k < p->ops[j].n_in; ++k)
        if (p->ops[j].in[k] == tv) v_read = true;
  const bool drop_v = !v_read && p->tensors[tv].role == GTF_ROLE_TMP;
  std::vector<OpInfo> ops;
  std::vector<int> origin, copies;
  for (int j = 0; j < n; ++j) {
    if (is_target[j]) {
      OpInfo c = p->ops[v];
      c.out = new_t[j];
      copies.push_back((int)ops.size());
      ops.push_back(c);
      origin.push_back(p->origin[v]);
      OpInfo r = p->ops[j];
      for (int k = 0; k < r.n_in; ++k)
        if (r.in[k] == tv) r.in[k] = new_t[j];
      ops.push_back(r);
      origin.push_back(p->origin[j]);
    } else if (!(j == v && drop_v)) {
      ops.push_back(p->ops[j]);
      origin.push_back(p->origin[j]);
    }
  }
  p->ops.swap(ops);
  p->origin.swap(origin);
  annotate(p);
  return copies;
}

// Duplicate fusion (DisCo, the fusion approach for a predecessor with
// several successors): an elementwise or broadcast op whose value crosses
// into other groups is recomputed inside each of those readers' groups
// instead of being stored and read back.  Ops are tried in program order;
// a duplication is kept when every copy lands in its reader's group and
// the plan's (HBM bytes, launches) strictly drops, and the scan then starts
// over; an op whose duplication is not kept is not tried again.  "Lands"
// means no copy's value is ever stored: every reader of every copy, this
// rewrite's or an earlier one's, shares the copy's group.
void duplicate_pass(FusePlan* p, bool row_resident) {
  std::set<int> blocked;  // descriptor op ids
  for (;;) {
    const auto gl = partition_groups(*p, true, row_resident);
    const auto cost = plan_cost(*p, gl);
    std::vector<int> gof(p->ops.size(), -1);
    for (size_t g = 0; g < gl.size(); ++g)
      for (int i : gl[g]) gof[i] = (int)g;
    const auto rd = readers_of(*p);
    bool kept = false;
    for (int v = 0; v < (int)p->ops.size() && !kept; ++v) {
      if (blocked.count(p->origin[v]) || p->ops[v].pattern > GTF_PAT_BROADCAST) continue;
      if (rd[v].size() < 2) continue;
      std::vector<int> targets;
      for (int r : rd[v])
        if (gof[r] != gof[v] && p->ops[r].pattern != GTF_PAT_OPAQUE) targets.push_back(r);
      if (targets.empty()) continue;
      FusePlan q = *p;
      const std::vector<int> copies = duplicate_op(&q, v, targets);
      const auto gl2 = partition_groups(q, true, row_resident);
      std::vector<int> gof2(q.ops.size(), -1);
      for (size_t g = 0; g < gl2.size(); ++g)
        for (int i : gl2[g]) gof2[i] = (int)g;
      // no value of a copy (this rewrite's or an earlier one's) is stored:
      // every reader of a copy shares the copy's group
      bool fused = !copies.empty();
      std::vector<int> prod(q.tensors.size(), -1);
      for (size_t i = 0; i < q.ops.size(); ++i) prod[q.ops[i].out] = (int)i;
      for (size_t j = 0; j < q.ops.size(); ++j)
        for (int k = 0; k < q.ops[j].n_in; ++k) {
          const int t = q.ops[j].in[k];
          if (t >= q.n_desc_tensors && gof2[prod[t]] != gof2[j]) fused = false;
        }
      if (fused && plan_cost(q, gl2) < cost) {
        *p = std::move(q);
        kept = true;
      } else {
        blocked.insert(p->origin[v]);
      }
    }
    if (!kept) return;
  }
}

}  // namespace

namespace {
void init_origin(FusePlan* p) {
  if (p->origin.size() != p->ops.size()) {
    p->n_desc_ops = (int)p->ops.size();
    p->n_desc_tensors = (int)p->tensors.size();
    p->origin.resize(p->ops.size());
    for (size_t i = 0; i < p->ops.size(); ++i) p->origin[i] = (int)i;
  }
}
}  // namespace

int build_fuse_plan(FusePlan* p, bool fuse, bool row_resident, bool duplicate) {
  init_origin(p);
  annotate(p);
  if (fuse && duplicate) duplicate_pass(p, row_resident);
  return finish_plan(p, partition_groups(*p, fuse, row_resident));
}

// Order the groups by their dependencies, compile each, and mark the
// tensors that go through memory.
int finish_plan(FusePlan* p, const std::vector<std::vector<int>>& gl) {
  std::vector<int> gpat;
  for (const auto& g : gl) {
    int pat = 0;
    for (int i : g) pat = std::max(pat, p->ops[i].pattern);
    gpat.push_back(pat);
  }
  std::vector<int> owner(p->tensors.size(), -1);
  for (size_t g = 0; g < gl.size(); ++g)
    for (int i : gl[g]) owner[p->ops[i].out] = (int)g;
  std::vector<std::set<int>> deps(gl.size());
  for (size_t g = 0; g < gl.size(); ++g)
    for (int i : gl[g])
      for (int k = 0; k < p->ops[i].n_in; ++k) {
        int o = owner[p->ops[i].in[k]];
        if (o >= 0 && o != (int)g) deps[g].insert(o);
      }
  std::vector<char> placed(gl.size(), 0);
  p->groups.clear();
  for (size_t step = 0; step < gl.size(); ++step) {
    int pick = -1;
    for (size_t g = 0; g < gl.size(); ++g) {
      if (placed[g]) continue;
      bool r = true;
      for (int d : deps[g])
        if (!placed[d]) r = false;
      if (r && (pick < 0 || gl[g][0] < gl[pick][0])) pick = (int)g;
    }
    if (pick < 0) return fail(GTF_E_INVALID, "groups depend on each other in a cycle");
    placed[pick] = 1;
    Group G;
    G.ops = gl[pick];
    G.pattern = gpat[pick];
    std::string why;
    if (!compile_group(*p, G.ops, &G.code, &why))
      return fail(GTF_E_LIMIT, "group of op " + std::to_string(G.ops[0]) + ": " + why);
    p->groups.push_back(G);
  }
  // materialised tensors
  p->materialized.assign(p->tensors.size(), 0);
  for (size_t t = 0; t < p->tensors.size(); ++t)
    if (p->tensors[t].role != GTF_ROLE_TMP) p->materialized[t] = 1;
  std::vector<int> gof(p->tensors.size(), -1);
  for (size_t g = 0; g < p->groups.size(); ++g)
    for (int i : p->groups[g].ops) gof[p->ops[i].out] = (int)g;
  for (size_t g = 0; g < p->groups.size(); ++g)
    for (int i : p->groups[g].ops)
      for (int k = 0; k < p->ops[i].n_in; ++k) {
        int t = p->ops[i].in[k];
        if (gof[t] >= 0 && gof[t] != (int)g) p->materialized[t] = 1;
      }
  // the caller provides memory for descriptor tensors only
  for (const Group& G : p->groups)
    for (int t : G.code.slot_tensor)
      if (t >= p->n_desc_tensors) return fail(GTF_E_LIMIT, "an internal tensor would be stored");
  if (std::getenv("GTF_TRACE")) {
    for (size_t g = 0; g < p->groups.size(); ++g) {
      const Group& G = p->groups[g];
      std::fprintf(stderr, "[gtf] group %zu pattern %d ops", g, G.pattern);
      for (int i : G.ops) std::fprintf(stderr, " %d", i);
      const ExecArgs& a = G.code.args;
      std::fprintf(stderr, " | dom %lldx%lld items %lld PW %d RB %d tpr %d K %d NS %d col %d stages %d depth %d\n",
                   (long long)a.R, (long long)a.C, (long long)a.n_items, a.PW, a.RB,
                   1 << a.tpr_log2, a.K, a.NS, a.n_col, a.n_stages, G.code.max_depth);
      for (int st = 0; st < a.n_stages; ++st)
        std::fprintf(stderr, "    stage %d: row %d+%d elem %d+%d red %d lds %d slot %d\n", st,
                     a.stage[st].row_off, a.stage[st].row_len, a.stage[st].el_off, a.stage[st].el_len,
                     a.stage[st].red, a.stage[st].red_lds, a.stage[st].red_slot);
      int tot = a.stage[a.n_stages - 1].el_off + a.stage[a.n_stages - 1].el_len;
      for (int k = 0; k < tot; ++k)
        std::fprintf(stderr, "    %3d form %2d arg %d imm %g\n", k, a.prog[k].code, a.prog[k].arg,
                     a.prog[k].imm);
    }
  }
  return GTF_OK;
}

// ================================================================ explicit groupings and search
namespace {

// Groups from per-op labels, in order of each label's first op.
std::vector<std::vector<int>> groups_from_labels(const std::vector<int>& labels) {
  std::vector<std::vector<int>> gl;
  std::map<int, int> index;
  for (size_t i = 0; i < labels.size(); ++i) {
    auto it = index.find(labels[i]);
    if (it == index.end()) {
      index[labels[i]] = (int)gl.size();
      gl.push_back({(int)i});
    } else {
      gl[it->second].push_back((int)i);
    }
  }
  return gl;
}

// A valid plan: an acyclic group graph (so every group is convex), every
// group within the op limit and compilable (argument limit, shapes, stages
// and the kernel's resources).
bool plan_ok(const FusePlan& p, const std::vector<int>& labels, std::string* why) {
  const auto gl = groups_from_labels(labels);
  std::map<int, int> gidx;
  for (size_t g = 0; g < gl.size(); ++g) gidx[labels[gl[g][0]]] = (int)g;
  for (const auto& g : gl) {
    if ((int)g.size() > GTF_MAX_GROUP_OPS) {
      if (why) *why = "group over the op limit";
      return false;
    }
    // DisCo's plans never fuse a parameter or control-flow op: an opaque op
    // stays a group of its own
    if (g.size() > 1)
      for (int i : g)
        if (p.ops[i].pattern == GTF_PAT_OPAQUE) {
          if (why) *why = "an opaque op is fused with others";
          return false;
        }
    if (!compile_group(p, g, nullptr, why)) return false;
  }
  std::vector<int> owner(p.tensors.size(), -1);
  for (size_t i = 0; i < p.ops.size(); ++i) owner[p.ops[i].out] = gidx[labels[i]];
  std::vector<std::set<int>> succ(gl.size());
  for (size_t j = 0; j < p.ops.size(); ++j)
    for (int k = 0; k < p.ops[j].n_in; ++k) {
      const int o = owner[p.ops[j].in[k]];
      const int gj = gidx[labels[j]];
      if (o >= 0 && o != gj) succ[o].insert(gj);
    }
  std::vector<int> indeg(gl.size(), 0);
  for (const auto& ss : succ)
    for (int b : ss) ++indeg[b];
  std::vector<int> ready;
  for (size_t g = 0; g < gl.size(); ++g)
    if (indeg[g] == 0) ready.push_back((int)g);
  size_t seen = 0;
  while (!ready.empty()) {
    const int a = ready.back();
    ready.pop_back();
    ++seen;
    for (int b : succ[a])
      if (--indeg[b] == 0) ready.push_back(b);
  }
  if (seen != gl.size()) {
    if (why) *why = "groups depend on each other in a cycle";
    return false;
  }
  return true;
}

// SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): a Weyl sequence mixed by two xor-shift-multiply
// rounds; below(n) is the next output modulo n.
struct SplitMix64 {
  uint64_t state;
  explicit SplitMix64(uint64_t seed) : state(seed) {}
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int below(int n) { return (int)(next() % (uint64_t)n); }
};

struct SearchState {
  FusePlan prog;            // ops, tensors, origin (no groups)
  std::vector<int> labels;  // group label per op
};

std::vector<int> predecessors(const FusePlan& p, int v) {
  std::vector<int> prod(p.tensors.size(), -1);
  for (size_t i = 0; i < p.ops.size(); ++i) prod[p.ops[i].out] = (int)i;
  std::set<int> ps;
  for (int k = 0; k < p.ops[v].n_in; ++k)
    if (prod[p.ops[v].in[k]] >= 0) ps.insert(prod[p.ops[v].in[k]]);
  return std::vector<int>(ps.begin(), ps.end());
}

int readers_of_tensor(const FusePlan& p, int t) {
  int n = 0;
  for (const OpInfo& o : p.ops) {
    bool reads = false;
    for (int k = 0; k < o.n_in; ++k)
      if (o.in[k] == t) reads = true;
    n += reads;
  }
  return n;
}

// Copy op pi right before op v; v reads the copy, which joins v's group.
SearchState with_copy(const SearchState& s, int pi, int v) {
  SearchState c;
  c.prog.n_desc_ops = s.prog.n_desc_ops;
  c.prog.n_desc_tensors = s.prog.n_desc_tensors;
  c.prog.tensors = s.prog.tensors;
  TensorInfo ti = s.prog.tensors[s.prog.ops[pi].out];
  ti.role = GTF_ROLE_TMP;
  c.prog.tensors.push_back(ti);
  const int nt = (int)c.prog.tensors.size() - 1;
  for (size_t j = 0; j < s.prog.ops.size(); ++j) {
    if ((int)j == v) {
      OpInfo cp = s.prog.ops[pi];
      cp.out = nt;
      c.prog.ops.push_back(cp);
      c.prog.origin.push_back(s.prog.origin[pi]);
      c.labels.push_back(s.labels[v]);
      OpInfo r = s.prog.ops[v];
      for (int k = 0; k < r.n_in; ++k)
        if (r.in[k] == s.prog.ops[pi].out) r.in[k] = nt;
      c.prog.ops.push_back(r);
    } else {
      c.prog.ops.push_back(s.prog.ops[j]);
    }
    c.prog.origin.push_back(s.prog.origin[j]);
    c.labels.push_back(s.labels[j]);
  }
  annotate(&c.prog);
  return c;
}

// One application of DisCo's method (i) (dup false: non-duplicate fusion)
// or (ii) (dup true: duplicate fusion).  v is drawn over the ops that have
// a predecessor op in another group, p over those predecessors (both in
// program order).  A move whose result is not a valid plan is not applied.
void fuse_move(SearchState* s, SplitMix64* rng, bool dup) {
  // v: an op with a predecessor op in another group; p: one of those
  const int n = (int)s->prog.ops.size();
  std::vector<std::vector<int>> cross(n);
  std::vector<int> eligible;
  for (int v = 0; v < n; ++v) {
    for (int q : predecessors(s->prog, v))
      if (s->labels[q] != s->labels[v]) cross[v].push_back(q);
    if (!cross[v].empty()) eligible.push_back(v);
  }
  if (eligible.empty()) return;
  const int v = eligible[rng->below((int)eligible.size())];
  const int pi = cross[v][rng->below((int)cross[v].size())];
  if (dup && readers_of_tensor(s->prog, s->prog.ops[pi].out) > 1) {
    SearchState c = with_copy(*s, pi, v);
    if (plan_ok(c.prog, c.labels, nullptr)) *s = std::move(c);
  } else {
    std::vector<int> lab = s->labels;
    const int lp = lab[pi], lv = lab[v];
    for (int& x : lab)
      if (x == lp) x = lv;
    if (plan_ok(s->prog, lab, nullptr)) s->labels.swap(lab);
  }
}

// A plan's identity: its program and its grouping, labels renumbered in
// order of first appearance.
std::string state_key(const SearchState& s) {
  std::string k;
  auto put = [&](const void* d, size_t n) { k.append((const char*)d, n); };
  for (const OpInfo& o : s.prog.ops) {
    put(&o.opcode, sizeof o.opcode);
    put(&o.n_in, sizeof o.n_in);
    put(o.in, sizeof o.in);
    put(&o.out, sizeof o.out);
    put(&o.imm, sizeof o.imm);
    put(&o.flags, sizeof o.flags);
  }
  std::map<int, int> ren;
  for (int x : s.labels) {
    auto it = ren.find(x);
    const int r = it == ren.end() ? (ren[x] = (int)ren.size()) : it->second;
    put(&r, sizeof r);
  }
  return k;
}

}  // namespace

int build_grouped_plan(FusePlan* p, const std::vector<int>& labels) {
  init_origin(p);
  annotate(p);
  if (labels.size() != p->ops.size()) return fail(GTF_E_INVALID, "one group label per op");
  for (int x : labels)
    if (x < 0) return fail(GTF_E_INVALID, "group labels must be >= 0");
  std::string why;
  if (!plan_ok(*p, labels, &why)) return fail(GTF_E_INVALID, "grouping not runnable: " + why);
  return finish_plan(p, groups_from_labels(labels));
}

// DisCo's backtracking search (its "Strategy Maker"): a queue of candidate
// plans ordered by cost (ties by insertion order), initially the program
// with every op its own launch.  Each step dequeues the cheapest, and for
// method (i) and then method (ii) applies that method to it n times (n drawn
// from 0..beta), costs the result once, keeps it as the best when cheaper,
// and enqueues it when its cost is at most alpha times the best.  Ends when the queue is empty, the
// best has not changed for max_stall steps, or after max_steps steps (0: no
// bound).  Method (iii), combining AllReduce instructions, has nothing to
// act on with one GPU.
int search_plan(FusePlan* p, const SearchParams& prm,
                const std::function<double(const FusePlan&)>& cost, SearchStats* st) {
  init_origin(p);
  annotate(p);
  if (!(prm.alpha >= 1.0) || prm.beta < 0 || prm.max_stall < 1 || prm.max_steps < 0)
    return fail(GTF_E_INVALID, "search parameters: alpha >= 1, beta >= 0, max_stall >= 1");
  SplitMix64 rng(prm.seed);
  std::vector<SearchState> states;
  SearchState start;
  start.prog.tensors = p->tensors;
  start.prog.ops = p->ops;
  start.prog.origin = p->origin;
  start.prog.n_desc_ops = p->n_desc_ops;
  start.prog.n_desc_tensors = p->n_desc_tensors;
  start.prog.ipdom = p->ipdom;
  for (size_t i = 0; i < p->ops.size(); ++i) start.labels.push_back((int)i);
  auto evaluate = [&](const SearchState& s, double* c) -> int {
    FusePlan fp = s.prog;
    int rc = finish_plan(&fp, groups_from_labels(s.labels));
    if (rc != GTF_OK) return rc;
    *c = cost(fp);
    if (!(*c >= 0.0)) return fail(GTF_E_INVALID, "cost callback returned a negative or NaN cost");
    return GTF_OK;
  };
  double c0 = 0.0;
  int rc = evaluate(start, &c0);
  if (rc != GTF_OK) return rc;
  states.push_back(start);
  typedef std::pair<double, int64_t> Key;  // (cost, insertion tick); the state index is the tick
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> queue;
  queue.push({c0, 0});
  std::set<std::string> seen{state_key(start)};
  SearchState best_state = start;
  int64_t stall = 0, steps = 0, evals = 0;
  double c_best = c0;
  while (!queue.empty() && stall < prm.max_stall && (prm.max_steps == 0 || steps < prm.max_steps)) {
    const int64_t h = queue.top().second;
    queue.pop();
    ++steps;
    bool improved = false;
    for (int dup = 0; dup < 2; ++dup) {
      SearchState cand = states[h];
      const int n = rng.below(prm.beta + 1);
      for (int k = 0; k < n; ++k) fuse_move(&cand, &rng, dup != 0);
      double cc = 0.0;
      rc = evaluate(cand, &cc);
      if (rc != GTF_OK) return rc;
      ++evals;
      if (cc < c_best) {
        c_best = cc;
        improved = true;
        best_state = cand;
      }
      // a plan enqueued before is not enqueued again
      if (cc <= prm.alpha * c_best && seen.insert(state_key(cand)).second) {
        queue.push({cc, (int64_t)states.size()});
        states.push_back(std::move(cand));
      }
    }
    stall = improved ? 0 : stall + 1;
  }
  if (st) {
    st->steps = steps;
    st->evaluations = evals;
    st->queue_left = (int64_t)queue.size();
    st->start_cost = c0;
    st->best_cost = c_best;
  }
  const SearchState& b = best_state;
  FusePlan out = b.prog;
  rc = finish_plan(&out, groups_from_labels(b.labels));
  if (rc != GTF_OK) return rc;
  *p = std::move(out);
  return GTF_OK;
}

}  // namespace gtf
