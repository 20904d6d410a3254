"""Plain data description of an op graph: tensors and ops, nothing computed.

A graph is what both the product (through its C-ABI binding) and the oracle
consume.  It is a list of tensors (name, dtype, shape, role) and a list of ops
in topological order, each op naming its input tensors and its one output
tensor.  Op names are strings; each side keeps its own table of what a name
means.

Roles: "in" (graph input, never written), "out" (graph output, written by
exactly one op; may also be read by later ops) and "tmp" (intermediate,
written by exactly one op and read by at least one later op).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

DTYPES = ("f32", "bf16", "u8")
ROLES = ("in", "out", "tmp")

# Op vocabulary with input counts.  Shapes broadcast NumPy-style over at most
# two axes: an operand is [R,C], [1,C] (or rank-1 [C]), [R,1] or [1,1].
OP_ARITY = {
    "copy": 1, "exp": 1, "tanh": 1, "sigmoid": 1, "relu": 1, "gelu": 1,
    "square": 1, "sqrt": 1, "recip": 1, "neg": 1,
    "add_imm": 1, "mul_imm": 1,
    "add": 2, "sub": 2, "mul": 2, "div": 2, "max": 2, "min": 2,
    "add3": 3, "dmul": 2,
    "row_sum": 1, "row_mean": 1, "row_max": 1,
    # injective data movement: [R,C] -> [C,R]; any shape to any shape of
    # the same element count (row-major order kept); [R,C1] ++ [R,C2] along
    # the last axis.  A tuple groups two [R,Ci] fields; its one reader is a
    # concat of that tuple alone (one input), which joins the fields the
    # same way.  Concat takes two tensors or one tuple.
    "transpose": 1, "reshape": 1, "concat": 2, "tuple": 2,
}


@dataclass(frozen=True)
class TensorDesc:
    name: str
    dtype: str
    shape: Tuple[int, ...]
    role: str


@dataclass(frozen=True)
class OpDesc:
    op: str
    inputs: Tuple[int, ...]
    output: int
    imm: float = 0.0
    opaque: bool = False


@dataclass
class Graph:
    tensors: List[TensorDesc] = field(default_factory=list)
    ops: List[OpDesc] = field(default_factory=list)

    # -- building helpers -------------------------------------------------
    def tensor(self, name: str, dtype: str, shape: Sequence[int], role: str) -> int:
        assert dtype in DTYPES and role in ROLES, (dtype, role)
        self.tensors.append(TensorDesc(name, dtype, tuple(int(s) for s in shape), role))
        return len(self.tensors) - 1

    def input(self, name: str, dtype: str, shape: Sequence[int]) -> int:
        return self.tensor(name, dtype, shape, "in")

    def op(self, op: str, inputs: Sequence[int], name: str, dtype: str,
           shape: Sequence[int], role: str = "tmp", imm: float = 0.0,
           opaque: bool = False) -> int:
        assert op in OP_ARITY, op
        out = self.tensor(name, dtype, shape, role)
        self.ops.append(OpDesc(op, tuple(inputs), out, float(imm), bool(opaque)))
        return out

    # -- queries ----------------------------------------------------------
    def producer(self, t: int) -> Optional[int]:
        for i, o in enumerate(self.ops):
            if o.output == t:
                return i
        return None

    def inputs(self) -> List[int]:
        return [i for i, t in enumerate(self.tensors) if t.role == "in"]

    def outputs(self) -> List[int]:
        return [i for i, t in enumerate(self.tensors) if t.role == "out"]
