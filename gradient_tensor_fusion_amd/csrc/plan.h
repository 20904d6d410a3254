// plan.h -- host-side fusion plan and bucket plan (internal).
#pragma once

#include <stdint.h>

#include <functional>
#include <string>
#include <vector>

#include "isa.h"

namespace gtf {

// Set the thread's last-error message and return the status.
int fail(int status, const std::string& msg);

struct TensorInfo {
  int dtype = 0, rank = 0, role = 0;
  int64_t R = 0, C = 0;   // normalised 2-D shape ([N] -> [1, N])
};

struct OpInfo {
  int opcode = 0, n_in = 0;
  int in[3] = {-1, -1, -1};
  int out = -1;
  float imm = 0.f;
  int flags = 0;
  int pattern = 0;
};

// A group compiled into an op-program plus its launch geometry.
struct CompiledGroup {
  ExecArgs args;                 // pointers filled per run
  std::vector<int> slot_tensor;  // external slot -> tensor id
  std::vector<int64_t> slot_numel;  // elements of each external tensor
  std::vector<int> slot_dtype;      // GTF_F32 / GTF_BF16 / GTF_U8 of each
  int n_slots = 0;
  int lds_bytes = 0;
  int max_depth = 0;
};

struct Group {
  std::vector<int> ops;  // ascending op ids
  int pattern = 0;
  CompiledGroup code;
};

struct FusePlan {
  // The program: the descriptor's tensors and ops, plus (with duplicate
  // fusion) internal tensors after them and copies of ops among them.
  std::vector<TensorInfo> tensors;
  std::vector<OpInfo> ops;
  std::vector<int> origin;       // per op: the descriptor op it computes
  int n_desc_ops = 0, n_desc_tensors = 0;
  std::vector<int> ipdom;        // -1: none
  std::vector<Group> groups;     // in run order
  std::vector<char> materialized;
};

// Range check of a compiled program's slot, LDS and spill indices; null
// when every index is inside what the launch provides.
const char* check_program(const ExecArgs& a, int n_slots);

// Compile a set of ops (ascending ids) into an op-program.  Returns false,
// with a reason, when the group does not fit the kernel's resources.
bool compile_group(const FusePlan& p, const std::vector<int>& ops, CompiledGroup* out,
                   std::string* why);

int build_fuse_plan(FusePlan* p, bool fuse, bool row_resident = false, bool duplicate = false);

// Order the groups (member lists) by their dependencies, compile each and
// mark the tensors that go through memory.
int finish_plan(FusePlan* p, const std::vector<std::vector<int>>& groups);

// A plan from an explicit grouping (one label per op; equal labels share a
// group), refused unless the group graph is acyclic and every group runs.
int build_grouped_plan(FusePlan* p, const std::vector<int>& labels);

struct SearchParams {
  double alpha = 1.05;
  int beta = 10;
  int max_stall = 1000;
  uint64_t seed = 0;
  int max_steps = 0;
};
struct SearchStats {
  int64_t steps = 0, evaluations = 0, queue_left = 0;
  double start_cost = 0.0, best_cost = 0.0;
};

// DisCo's backtracking search over fusion plans; on success *p is the best
// plan found (its program may hold duplicated ops).
int search_plan(FusePlan* p, const SearchParams& prm,
                const std::function<double(const FusePlan&)>& cost, SearchStats* st);

struct BucketPlan {
  int dtype = 0;
  int64_t cap_bytes = 0;
  std::vector<int64_t> numel;
  std::vector<int32_t> bucket_of;
  std::vector<int64_t> offset;
  std::vector<int64_t> bucket_numel;
  // launches: tensor range [t0, t1), bucket range [b0, b1], chunk range
  struct Launch {
    int t0, t1, b0, b1;
    int64_t c0, c1;
  };
  std::vector<Launch> launches;
  std::vector<Chunk> chunks;
  void* workspace = nullptr;     // where the chunk table was bound
};

int build_bucket_plan(BucketPlan* b);

}  // namespace gtf
