"""Fused operator groups and tensor-fusion buckets on one AMD Instinct MI355X.

Thin Python layer over libgtf.so (include/gtf.h); PyTorch supplies device
memory and streams.  Planning (OpPatternKind annotation, post-dominator
tree, grouping, op-program compilation, bucket planning) and every kernel
run in the native library.

    plan = FusePlan(graph)             # graph: .tensors and .ops (see below)
    plan.run({tensor_id: torch_tensor, ...})
    bp = BucketPlan(numel, cap_bytes=25 << 20)
    bp.bind(torch.empty(bp.workspace_bytes, dtype=torch.uint8, device="cuda"))
    bp.pack(grads, buckets, scale=1 / world_size)

A graph is any object with ``tensors`` (each with name, dtype in
{"f32","bf16","u8"}, shape, role in {"in","out","tmp"}) and ``ops`` (each
with op name, inputs, output, imm, opaque), ops in topological order.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_int64, c_size_t, c_void_p
from typing import Dict, List, Sequence

from . import _capi as C
from ._capi import GtfError

__all__ = ["FusePlan", "FuseMulti", "BucketPlan", "device_copy", "stream_probe", "search", "GtfError",
           "PATTERN_NAMES"]

PATTERN_NAMES = {0: "kElemWise", 1: "kBroadcast", 2: "kInjective", 3: "kCommReduce",
                 4: "kOutEWiseFusable", 7: "kTuple", 8: "kOpaque"}


def _program_desc(graph):
    nt, no = len(graph.tensors), len(graph.ops)
    tens = (C.TensorDesc * max(1, nt))()
    for i, t in enumerate(graph.tensors):
        d = tens[i]
        d.dtype = C.DTYPE[t.dtype]
        d.rank = len(t.shape)
        for k, s in enumerate(t.shape[:2]):
            d.shape[k] = int(s)
        d.role = C.ROLE[t.role]
        d.reserved = 0
    ops = (C.OpDesc * max(1, no))()
    for i, o in enumerate(graph.ops):
        d = ops[i]
        d.opcode = C.OPCODE[o.op]
        d.n_in = len(o.inputs)
        for k, t in enumerate(o.inputs[:3]):
            d.inp[k] = int(t)
        d.out = int(o.output)
        d.imm = float(o.imm)
        d.flags = C.OPF_OPAQUE if getattr(o, "opaque", False) else 0
    desc = C.ProgramDesc(C.ABI_VERSION, nt, tens, no, ops)
    return desc, tens, ops


class FusePlan:
    """fuse_plan_create and friends."""

    def __init__(self, graph, fuse: bool = True, row_resident: bool = False,
                 duplicate: bool = False):
        self.graph = graph
        self.n_tensors = len(graph.tensors)
        desc, self._tens, self._ops = _program_desc(graph)
        h = c_void_p()
        flags = ((0 if fuse else C.NO_FUSE) | (C.ROW_RESIDENT if row_resident else 0)
                 | (C.DUPLICATE if duplicate else 0))
        C.check(C.lib().fuse_plan_create(byref(desc), flags, byref(h)))
        self._h = h
        n = c_int32()
        C.check(C.lib().fuse_plan_num_ops(self._h, byref(n)))
        self.n_ops = n.value  # ops of the plan's program (copies included)

    @classmethod
    def _adopt(cls, graph, h, keep) -> "FusePlan":
        self = cls.__new__(cls)
        self.graph = graph
        self.n_tensors = len(graph.tensors)
        self._tens, self._ops = keep
        self._h = h
        n = c_int32()
        C.check(C.lib().fuse_plan_num_ops(self._h, byref(n)))
        self.n_ops = n.value
        return self

    @classmethod
    def grouped(cls, graph, group_of: Sequence[int]) -> "FusePlan":
        """fuse_plan_create_grouped: ops with equal labels form one group."""
        desc, tens, ops = _program_desc(graph)
        arr = (c_int32 * max(1, len(graph.ops)))(*[int(x) for x in group_of])
        h = c_void_p()
        C.check(C.lib().fuse_plan_create_grouped(byref(desc), arr, byref(h)))
        return cls._adopt(graph, h, (tens, ops))

    def program(self):
        """fuse_plan_program: the plan's program as a Graph (the graph's
        tensors, then internal ones named "~<id>"; its ops in run order)."""
        from workloads.graph import Graph, OpDesc, TensorDesc
        nt, no = c_int32(), c_int32()
        C.check(C.lib().fuse_plan_program(self._h, None, 0, byref(nt), None, 0, byref(no)))
        tens = (C.TensorDesc * max(1, nt.value))()
        ops = (C.OpDesc * max(1, no.value))()
        C.check(C.lib().fuse_plan_program(self._h, tens, nt.value, byref(nt), ops, no.value,
                                          byref(no)))
        dt = {v: k for k, v in C.DTYPE.items()}
        rl = {v: k for k, v in C.ROLE.items()}
        op_names = {v: k for k, v in C.OPCODE.items()}
        g = Graph()
        for t in range(nt.value):
            d = tens[t]
            name = self.graph.tensors[t].name if t < self.n_tensors else f"~{t}"
            g.tensors.append(TensorDesc(name, dt[d.dtype], tuple(int(d.shape[k]) for k in range(d.rank)),
                                        rl[d.role]))
        for i in range(no.value):
            d = ops[i]
            g.ops.append(OpDesc(op_names[d.opcode], tuple(int(d.inp[k]) for k in range(d.n_in)),
                                int(d.out), float(d.imm), bool(d.flags & C.OPF_OPAQUE)))
        return g

    def op_origin(self) -> List[int]:
        """Per program op, the graph op it computes."""
        arr = (c_int32 * max(1, self.n_ops))()
        C.check(C.lib().fuse_plan_op_origin(self._h, arr))
        return list(arr[: self.n_ops])

    def __del__(self):
        h = getattr(self, "_h", None)
        # at interpreter exit the module's globals may already be gone; the
        # process frees the plan then anyway
        lib = getattr(C, "_lib", None) if C is not None else None
        if h is not None and h.value and lib is not None:
            lib.fuse_plan_destroy(h)
            self._h = None

    @property
    def num_groups(self) -> int:
        n = c_int32()
        C.check(C.lib().fuse_plan_num_groups(self._h, byref(n)))
        return n.value

    def group_ops(self, g: int) -> List[int]:
        n, pat = c_int32(), c_int32()
        C.check(C.lib().fuse_plan_group_info(self._h, g, None, 0, byref(n), byref(pat)))
        ids = (c_int32 * max(1, n.value))()
        C.check(C.lib().fuse_plan_group_info(self._h, g, ids, n.value, byref(n), byref(pat)))
        return list(ids[: n.value])

    def group_tensors(self, g: int) -> List[int]:
        """Tensors group g reads or writes in device memory, each once."""
        n = c_int32()
        C.check(C.lib().fuse_plan_group_tensors(self._h, g, None, 0, byref(n)))
        ids = (c_int32 * max(1, n.value))()
        C.check(C.lib().fuse_plan_group_tensors(self._h, g, ids, n.value, byref(n)))
        return list(ids[: n.value])

    def group_pattern(self, g: int) -> int:
        n, pat = c_int32(), c_int32()
        C.check(C.lib().fuse_plan_group_info(self._h, g, None, 0, byref(n), byref(pat)))
        return pat.value

    def groups(self) -> List[List[int]]:
        return [self.group_ops(g) for g in range(self.num_groups)]

    def op_info(self):
        pats = (c_int32 * max(1, self.n_ops))()
        ipd = (c_int32 * max(1, self.n_ops))()
        C.check(C.lib().fuse_plan_op_info(self._h, pats, ipd))
        return list(pats[: self.n_ops]), [None if v < 0 else v for v in ipd[: self.n_ops]]

    def geometry(self, g: int) -> dict:
        geo = C.GroupGeometry()
        C.check(C.lib().fuse_plan_group_geometry(self._h, g, byref(geo)))
        return {name: getattr(geo, name) for name, _ in C.GroupGeometry._fields_}

    def code(self, g: int) -> dict:
        """fuse_plan_group_code: group g's compiled op program (forms as
        numbers, stages, slot strides), for host-side checks of the group
        compiler."""
        info = C.GroupCode()
        C.check(C.lib().fuse_plan_group_code(self._h, g, byref(info), None, 0))
        code = (C.Instr * max(1, info.n_instr))()
        C.check(C.lib().fuse_plan_group_code(self._h, g, byref(info), code, info.n_instr))
        stages = [{n: getattr(info.stage[k], n) for n, _ in C.StageCode._fields_}
                  for k in range(info.n_stages)]
        return {"n_col": info.n_col, "stages": stages,
                "instr": [(int(code[i].form), int(code[i].arg), float(code[i].imm))
                          for i in range(info.n_instr)],
                "slots": self.group_tensors(g), "transposed_slot": info.transposed_slot,
                "rstride": list(info.rstride[:info.n_slots]),
                "cstride": list(info.cstride[:info.n_slots])}

    def is_materialized(self, t: int) -> bool:
        y = c_int32()
        C.check(C.lib().fuse_plan_is_materialized(self._h, t, byref(y)))
        return bool(y.value)

    def materialized(self) -> List[int]:
        return [t for t in range(self.n_tensors) if self.is_materialized(t)]

    def _tensor_bytes(self, t: int) -> int:
        d = self.graph.tensors[t]
        n = 1
        for s in d.shape:
            n *= int(s)
        return n * C.ELEM_BYTES[d.dtype]

    def _ptr(self, t: int, x):
        return C.device_ptr(x, self._tensor_bytes(t), f"tensor {t} ({self.graph.tensors[t].name})")

    def _ptrs(self, tensors) -> ctypes.Array:
        if isinstance(tensors, dict):
            ptrs = [self._ptr(t, tensors.get(t)) for t in range(self.n_tensors)]
        else:
            # the library reads one pointer per tensor of the graph
            if len(tensors) != self.n_tensors:
                raise ValueError(f"{len(tensors)} tensors for a graph of {self.n_tensors}")
            ptrs = [self._ptr(t, x) for t, x in enumerate(tensors)]
        return C.ptr_array(ptrs)

    def run_group(self, g: int, tensors, stream=None) -> None:
        C.check(C.lib().fuse_group_run(self._h, g, self._ptrs(tensors), C.stream_handle(stream)))

    def run(self, tensors, stream=None) -> None:
        C.check(C.lib().fuse_plan_run(self._h, self._ptrs(tensors), C.stream_handle(stream)))

    def launcher(self, g: int, tensors, stream=None):
        """fuse_group_run with its arguments marshalled once: returns a
        callable that launches group g on the same tensors and stream.  The
        stream is fixed here (the current one unless given), so a launcher
        made before a graph capture does not launch into the capture."""
        f, h, ptrs, st = C.lib().fuse_group_run, self._h, self._ptrs(tensors), C.stream_handle(stream)
        keep = tensors

        def run():
            status = f(h, g, ptrs, st)
            if status != C.GTF_OK:
                C.check(status)
        run.tensors = keep
        return run


class _Candidate(FusePlan):
    """A candidate plan handed to a search cost callback: borrowed, valid
    only during the call."""

    def __del__(self):
        pass


def search(graph, cost, alpha: float = 1.05, beta: int = 10, max_stall: int = 1000,
           seed: int = 0, max_steps: int = 0):
    """fuse_plan_search: DisCo's backtracking search over fusion plans.
    cost(candidate) gets a FusePlan valid only during the call (runnable on
    the graph's tensors) and returns its cost.  Returns (best FusePlan,
    stats dict)."""
    desc, tens, ops = _program_desc(graph)
    err = []

    def cb(_ctx, handle):
        try:
            cand = _Candidate._adopt(graph, c_void_p(handle), (tens, ops))
            return float(cost(cand))
        except BaseException as e:  # reported after the search stops
            err.append(e)
            return float("nan")
    fn = C.COST_FN(cb)
    prm = C.SearchParams(alpha, beta, max_stall, seed, max_steps, 0)
    st = C.SearchStats()
    h = c_void_p()
    status = C.lib().fuse_plan_search(byref(desc), byref(prm), fn, None, byref(h), byref(st))
    if err:
        raise err[0]
    C.check(status)
    stats = {name: getattr(st, name) for name, _ in C.SearchStats._fields_}
    return FusePlan._adopt(graph, h, (tens, ops)), stats


class FuseMulti:
    """fuse_multi_create / bind / run: one launch of a flat group over many
    tensor sets (set s: numel[s] elements per tensor)."""

    def __init__(self, plan: "FusePlan", g: int, numel: Sequence[int]):
        self.plan = plan  # the group's program lives in the plan's compiled copy; keep it alive
        self.numel = [int(n) for n in numel]
        arr = (c_int64 * max(1, len(self.numel)))(*self.numel)
        h = c_void_p()
        C.check(C.lib().fuse_multi_create(plan._h, int(g), len(self.numel), arr, byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        # at interpreter exit the module's globals may already be gone; the
        # process frees the plan then anyway
        lib = getattr(C, "_lib", None) if C is not None else None
        if h is not None and h.value and lib is not None:
            lib.fuse_multi_destroy(h)
            self._h = None

    @property
    def workspace_bytes(self) -> int:
        b = c_size_t()
        C.check(C.lib().fuse_multi_workspace_bytes(self._h, byref(b)))
        return b.value

    def bind(self, sets, workspace, stream=None) -> None:
        """sets: one {tensor id: tensor} dict per set."""
        nt = self.plan.n_tensors
        # the library reads one row of pointers per set it was created with
        if len(sets) != len(self.numel):
            raise ValueError(f"{len(sets)} tensor sets for a run of {len(self.numel)}")
        ptrs = []
        for s, d in enumerate(sets):
            for t in range(nt):
                el = C.ELEM_BYTES[self.plan.graph.tensors[t].dtype]
                ptrs.append(C.device_ptr(d.get(t), self.numel[s] * el, f"set {s} tensor {t}"))
        self._ws, self._sets = workspace, sets  # keep them alive while runs read them
        C.check(C.lib().fuse_multi_bind(self._h, C.ptr_array(ptrs),
                                        C.device_ptr(workspace, self.workspace_bytes, "workspace", True),
                                        C.stream_handle(stream)))

    def run(self, stream=None) -> None:
        C.check(C.lib().fuse_multi_run(self._h, C.stream_handle(stream)))

    def launcher(self, stream=None):
        f, h, st = C.lib().fuse_multi_run, self._h, C.stream_handle(stream)

        def run():
            status = f(h, st)
            if status != C.GTF_OK:
                C.check(status)
        return run


class BucketPlan:
    """bucket_plan_create / bind / pack / unpack."""

    def __init__(self, numel: Sequence[int], dtype: str = "f32", cap_bytes: int = 25 << 20):
        self.numel = [int(n) for n in numel]
        arr = (c_int64 * max(1, len(self.numel)))(*self.numel)
        h = c_void_p()
        C.check(C.lib().bucket_plan_create(arr, len(self.numel), C.DTYPE[dtype], int(cap_bytes), 0,
                                           byref(h)))
        self._h = h
        self.dtype = dtype
        self.cap_bytes = int(cap_bytes)
        self._bucket_numel = self.query()[2]

    def __del__(self):
        h = getattr(self, "_h", None)
        # at interpreter exit the module's globals may already be gone; the
        # process frees the plan then anyway
        lib = getattr(C, "_lib", None) if C is not None else None
        if h is not None and h.value and lib is not None:
            lib.bucket_plan_destroy(h)
            self._h = None

    def query(self):
        nb = c_int32()
        C.check(C.lib().bucket_plan_query(self._h, byref(nb), None, None, None))
        n = len(self.numel)
        bof = (c_int32 * max(1, n))()
        off = (c_int64 * max(1, n))()
        bn = (c_int64 * max(1, nb.value))()
        C.check(C.lib().bucket_plan_query(self._h, byref(nb), bof, off, bn))
        return list(bof[:n]), list(off[:n]), list(bn[: nb.value])

    @property
    def workspace_bytes(self) -> int:
        b = c_size_t()
        C.check(C.lib().bucket_plan_workspace_bytes(self._h, byref(b)))
        return b.value

    def bind(self, workspace, stream=None) -> None:
        self._ws = workspace  # keep it alive as long as the plan uses it
        C.check(C.lib().bucket_plan_bind(self._h, C.device_ptr(workspace, self.workspace_bytes, "workspace", True),
                                         C.stream_handle(stream)))

    def _tensor_ptrs(self, tensors) -> ctypes.Array:
        el = C.ELEM_BYTES[self.dtype]
        if len(tensors) != len(self.numel):
            raise ValueError(f"{len(tensors)} tensors for a plan of {len(self.numel)}")
        return C.ptr_array([C.device_ptr(x, n * el, f"tensor {i}")
                            for i, (x, n) in enumerate(zip(tensors, self.numel))])

    def _bucket_ptrs(self, buckets) -> ctypes.Array:
        el = C.ELEM_BYTES[self.dtype]
        if len(buckets) != len(self._bucket_numel):
            raise ValueError(f"{len(buckets)} buckets for a plan of {len(self._bucket_numel)}")
        return C.ptr_array([C.device_ptr(x, n * el, f"bucket {k}")
                            for k, (x, n) in enumerate(zip(buckets, self._bucket_numel))])

    def pack(self, srcs, buckets, scale: float = 1.0, stream=None) -> None:
        C.check(C.lib().bucket_pack(self._h, self._tensor_ptrs(srcs), self._bucket_ptrs(buckets),
                                    float(scale), C.stream_handle(stream)))

    def unpack(self, buckets, dsts, scale: float = 1.0, stream=None) -> None:
        C.check(C.lib().bucket_unpack(self._h, self._bucket_ptrs(buckets), self._tensor_ptrs(dsts),
                                      float(scale), C.stream_handle(stream)))

    def launcher(self, unpack: bool, tensors, buckets, scale: float, stream=None):
        """bucket_pack (or bucket_unpack) with its arguments marshalled once."""
        t = self._tensor_ptrs(tensors)
        b = self._bucket_ptrs(buckets)
        h, st, sc = self._h, C.stream_handle(stream), float(scale)
        keep = (tensors, buckets)
        if unpack:
            f, a0, a1 = C.lib().bucket_unpack, b, t
        else:
            f, a0, a1 = C.lib().bucket_pack, t, b

        def run():
            status = f(h, a0, a1, sc, st)
            if status != C.GTF_OK:
                C.check(status)
        run.tensors = keep
        return run

    def slot_address(self, buckets, i: int) -> int:
        """bucket_plan_slot_address: device address of tensor i in its bucket."""
        out = c_void_p()
        C.check(C.lib().bucket_plan_slot_address(self._h, self._bucket_ptrs(buckets),
                                                 int(i), byref(out)))
        return out.value or 0

    def slot_view(self, buckets, i: int, shape):
        """Tensor i's place in its bucket as a tensor view of the given shape
        (its data_ptr() is slot_address(buckets, i)): an output for a fused
        group whose stores then are the pack."""
        if not hasattr(self, "_layout"):
            self._layout = self.query()
        bof, off, _ = self._layout
        b = buckets[bof[i]]
        n = self.numel[i]
        v = b.reshape(-1).narrow(0, off[i], n).view(tuple(shape))
        assert n == 0 or v.data_ptr() == self.slot_address(buckets, i)
        return v

    def pack_per_tensor(self, srcs, buckets, scale: float = 1.0, stream=None) -> None:
        C.check(C.lib().bucket_pack_per_tensor(self._h, self._tensor_ptrs(srcs),
                                               self._bucket_ptrs(buckets),
                                               float(scale), C.stream_handle(stream)))

    def pack_static(self, srcs, buckets, scale: float = 1.0, stream=None) -> None:
        """bucket_pack_static: pack with the chunk table in the library's
        static device array (no workspace, no bind, allocates nothing)."""
        C.check(C.lib().bucket_pack_static(self._h, self._tensor_ptrs(srcs), self._bucket_ptrs(buckets),
                                           float(scale), C.stream_handle(stream)))

    def unpack_per_tensor(self, buckets, dsts, scale: float = 1.0, stream=None) -> None:
        C.check(C.lib().bucket_unpack_per_tensor(self._h, self._bucket_ptrs(buckets),
                                                 self._tensor_ptrs(dsts),
                                                 float(scale), C.stream_handle(stream)))


def stream_probe(kind: int, depth: int, nontemporal: bool, grid_per_cu: int, dst, src,
                 nbytes: int, stream=None) -> None:
    """gtf_stream_probe: copy (kind 0), read (1) or write (2) nbytes."""
    n = int(nbytes)
    sp = None if kind == 2 else C.device_ptr(src, n, "src", True)
    C.check(C.lib().gtf_stream_probe(int(kind), int(depth), int(bool(nontemporal)), int(grid_per_cu),
                                     C.device_ptr(dst, n, "dst", True), sp, n,
                                     C.stream_handle(stream)))


def device_copy(dst, src, nbytes: int, stream=None) -> None:
    n = int(nbytes)
    C.check(C.lib().gtf_device_copy(C.device_ptr(dst, n, "dst", True), C.device_ptr(src, n, "src", True), n,
                                    C.stream_handle(stream)))
