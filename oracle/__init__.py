"""The oracle: a plain, slow CPU implementation of what the fused-group
executor and the tensor-fusion buckets compute.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports, calls or links
anything here; only the test suite, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may use it.  It shares no code with
the HIP path: its op semantics, its pattern annotation, its post-dominator
computation, its grouping rule and its bucket planner are all written here,
separately, from the pages:

* Apache TVM, "Operator Fusion" (docs/arch/fusion.rst): the OpPatternKind
  table, the post-dominator grouping algorithm and its fusion rules, and the
  add/exp/squeeze example.
* Optimizing DNN Compilation for Distributed Training with Joint OP and
  Tensor Fusion (DisCo, arXiv 2209.12769), section 1: op fusion keeps
  intermediates out of device memory; tensor fusion concatenates small
  gradient tensors so the fused size is the sum of the sizes; AllReduce sums
  or averages gradients.

Modules
-------
numerics   bf16 / u8 decoding and fp32 -> bf16 round-to-nearest-even.
ops        what each op computes (fp32 IEEE ops, fp64 transcendentals).
evaluate   op-by-op unfused evaluation of a graph.
partition  pattern annotation, post-dominators, the grouping rule.
bucket     next-fit buckets, dense offsets, pack and unpack with a scale.
"""
