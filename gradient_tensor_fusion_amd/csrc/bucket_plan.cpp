// bucket_plan.cpp -- tensor-fusion bucket planning on the host.
//
// DisCo (arXiv 2209.12769), section 1: small gradient tensors are fused
// before the AllReduce and the fused tensor's size is the sum of the
// members' sizes; the combining is bounded by a size threshold (the XLA
// AllReduce combiner passage in section 1, Horovod's fusion threshold in
// section 7).  Buckets are filled next-fit in production order with dense
// offsets; the chunk table then cuts every tensor into runs of at most
// kChunkBytes bytes so one launch balances tensors of any size.
#include <algorithm>

#include "gtf.h"
#include "plan.h"

namespace gtf {

int build_bucket_plan(BucketPlan* b) {
  const int n = (int)b->numel.size();
  const int64_t eb = b->dtype == GTF_BF16 ? 2 : 4;
  b->bucket_of.assign(n, 0);
  b->offset.assign(n, 0);
  b->bucket_numel.clear();
  for (int i = 0; i < n; ++i) {
    const int64_t bytes = b->numel[i] * eb;
    bool fits = false;
    if (!b->bucket_numel.empty()) {
      const int64_t fill = b->bucket_numel.back() * eb;
      fits = fill + bytes <= b->cap_bytes || fill == 0;
    }
    if (!fits) b->bucket_numel.push_back(0);
    b->bucket_of[i] = (int32_t)b->bucket_numel.size() - 1;
    b->offset[i] = b->bucket_numel.back();
    b->bucket_numel.back() += b->numel[i];
  }
  // launches: consecutive tensors while tensors + buckets fit the pointer
  // table of one launch
  b->launches.clear();
  b->chunks.clear();
  int t0 = 0;
  while (t0 < n) {
    int t1 = t0;
    while (t1 < n) {
      const int b0 = b->bucket_of[t0], b1 = b->bucket_of[t1];
      if ((t1 + 1 - t0) + (b1 - b0 + 1) > kMaxBucketPtrs) break;
      ++t1;
    }
    BucketPlan::Launch L;
    L.t0 = t0;
    L.t1 = t1;
    L.b0 = b->bucket_of[t0];
    L.b1 = b->bucket_of[t1 - 1];
    L.c0 = (int64_t)b->chunks.size();
    const int nt = t1 - t0;
    const int64_t per_chunk = kChunkBytes / eb;
    for (int i = t0; i < t1; ++i) {
      for (int64_t s = 0; s < b->numel[i]; s += per_chunk) {
        Chunk c;
        c.t_off = s;
        c.b_off = b->offset[i] + s;
        c.n = (int32_t)std::min<int64_t>(per_chunk, b->numel[i] - s);
        c.t_slot = (uint16_t)(i - t0);
        c.b_slot = (uint16_t)(nt + (b->bucket_of[i] - L.b0));
        b->chunks.push_back(c);
      }
    }
    L.c1 = (int64_t)b->chunks.size();
    b->launches.push_back(L);
    t0 = t1;
  }
  return GTF_OK;
}

}  // namespace gtf
