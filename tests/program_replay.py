"""Host replay of the group compiler's output (no GPU): each group's op
program, as fuse_plan_group_code hands it over, run instruction by
instruction over whole arrays in NumPy, group after group as a run
launches them.

The replay restates what each instruction form does in the executor: two
working registers A and B and the spill slots hold one value each (a [1,C]
column in the column phase, an [R,1] column of row values in the row
phase, the [R,C] domain in the element phase); every op writes A, reading
A (and B, or an LDS slot, or an immediate), or B alone for the unary and
immediate forms that keep their operand in B; loads and stores address an
external tensor by phase (the element phase walks the domain in row-major
order, the row phase reads element r * rstride, the column phase element
c * cstride, and the addressed loads element r * rstride + c * cstride);
reductions fold A into the stage's accumulator, whose result goes to an
LDS row slot and/or an external tensor.

Arithmetic is fp32 for the IEEE operations, and correctly rounded from fp64
for the transcendentals and the reductions, so a replayed output matches
the oracle's evaluation to within the per-element bound the GPU tests use,
and bit for bit wherever only IEEE operations lead to it: what the replay
checks is the program's data flow (every operand the right value, every
result where the group's ops put it), which a wrong register, slot, form
or stage in a compiled program breaks."""
from __future__ import annotations

import re
from math import erf
from pathlib import Path
from typing import Dict

import numpy as np

from oracle import numerics

_ISA = Path(__file__).resolve().parent.parent / "gradient_tensor_fusion_amd" / "csrc" / "isa.h"


def _forms() -> Dict[str, int]:
    """The form enumeration of the executor's instruction set, by name."""
    text = _ISA.read_text()
    body = re.search(r"enum Form : int \{(.*?)\};", text, re.S).group(1)
    body = re.sub(r"//[^\n]*", "", body)
    names, n = {}, 0
    for item in body.replace("\n", " ").split(","):
        item = item.strip()
        if not item:
            continue
        if "=" in item:
            name, v = (x.strip() for x in item.split("="))
            n = int(v)
        else:
            name = item
        if name != "F_COUNT":
            names[name[2:]] = n
        n += 1
    return names


F = _forms()
NAME = {v: k for k, v in F.items()}
_XOPS = ["ADD", "SUB", "RSUB", "MUL", "DIV", "RDIV", "MAX", "MIN"]

_erf = np.vectorize(erf, otypes=[np.float64])


def _unary(name: str, x: np.ndarray) -> np.ndarray:
    d = x.astype(np.float64)
    with np.errstate(all="ignore"):
        if name == "EXP":
            y = np.exp(d)
        elif name == "TANH":
            y = np.tanh(d)
        elif name == "SIGMOID":
            y = 1.0 / (1.0 + np.exp(-d))
        elif name in ("GELU", "GELU_BF"):
            y = 0.5 * d * (1.0 + _erf(d / np.sqrt(2.0)))
        elif name == "RELU":
            return np.where(x > 0, x, np.float32(0)).astype(np.float32)
        elif name == "SQUARE":
            return (x * x).astype(np.float32)
        elif name == "SQRT":
            return np.sqrt(x).astype(np.float32)
        elif name == "RECIP":
            return (np.float32(1) / x).astype(np.float32)
        elif name == "NEG":
            return (-x).astype(np.float32)
        else:
            raise KeyError(name)
    return y.astype(np.float32)


def _xop(op: str, v, x) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32)
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(all="ignore"):
        r = {"ADD": lambda: v + x, "SUB": lambda: v - x, "RSUB": lambda: x - v,
             "MUL": lambda: v * x, "DIV": lambda: v / x, "RDIV": lambda: x / v,
             "MAX": lambda: np.fmax(v, x), "MIN": lambda: np.fmin(v, x)}[op]()
    return np.asarray(r, dtype=np.float32)


def _to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return numerics.bf16_to_f32(arr)
    return np.asarray(arr).astype(np.float32)


def _from_f32(vals: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return numerics.f32_to_bf16(vals.astype(np.float32))
    if dtype == "u8":
        raise AssertionError("the executor stores no u8 tensor")
    return vals.astype(np.float32)


class _Group:
    def __init__(self, graph, plan, g, mem):
        self.graph, self.mem = graph, mem
        self.code = plan.code(g)
        geo = plan.geometry(g)
        self.R, self.C = int(geo["rows"]), int(geo["cols"])
        self.slots = self.code["slots"]
        self.rs, self.cs = self.code["rstride"], self.code["cstride"]
        self.col_lds: Dict[int, np.ndarray] = {}
        self.row_lds: Dict[int, np.ndarray] = {}

    # ---- external tensors, as flat arrays of their element values
    def _flat(self, s: int) -> np.ndarray:
        t = self.slots[s]
        return _to_f32(self.mem[t], self.graph.tensors[t].dtype).ravel()

    def _store(self, s: int, idx: np.ndarray, vals: np.ndarray) -> None:
        t = self.slots[s]
        d = self.graph.tensors[t]
        flat = np.asarray(self.mem[t]).reshape(-1).copy()
        flat[idx.ravel()] = _from_f32(np.asarray(vals, dtype=np.float32).ravel(), d.dtype)
        self.mem[t] = flat.reshape(self.mem[t].shape)

    def _index(self, phase: str, s: int) -> np.ndarray:
        R, C = self.R, self.C
        if phase == "col":
            return (np.arange(C, dtype=np.int64) * self.cs[s]).reshape(1, C)
        if phase == "row":
            return (np.arange(R, dtype=np.int64) * self.rs[s]).reshape(R, 1)
        return np.arange(R * C, dtype=np.int64).reshape(R, C)

    def _addressed(self, s: int, c_shift: int = 0) -> np.ndarray:
        r = np.arange(self.R, dtype=np.int64).reshape(-1, 1)
        c = np.arange(self.C, dtype=np.int64).reshape(1, -1) - c_shift
        return r * self.rs[s] + c * self.cs[s]

    def _shape(self, phase: str):
        return {"col": (1, self.C), "row": (self.R, 1), "elem": (self.R, self.C)}[phase]

    # ---- one program of one phase
    def run(self, lo: int, n: int, phase: str, acc: list) -> None:
        shape = self._shape(phase)
        reg: Dict[str, np.ndarray] = {}

        def get(r):
            if r not in reg:
                raise AssertionError(f"{phase} program reads {r} before anything is put there")
            return reg[r]

        def lds(kind, arg):
            table = self.col_lds if kind == "C" else self.row_lds
            if arg not in table:
                raise AssertionError(f"{phase} program reads LDS {kind} slot {arg} before it is written")
            return table[arg]

        for pc in range(lo, lo + n):
            form, arg, imm = self.code["instr"][pc]
            name = NAME[form]
            m = re.fullmatch(r"LD_(F32|BF16|U8)_([AB])", name)
            if m:
                v = self._flat(arg)[self._index(phase, arg)]
                reg[m.group(2)] = np.broadcast_to(v, shape).astype(np.float32)
                continue
            m = re.fullmatch(r"(COL|ROW|IMM)_([AB])", name)
            if m:
                src = imm if m.group(1) == "IMM" else lds(m.group(1)[0], arg)
                reg[m.group(2)] = np.broadcast_to(np.float32(src) if m.group(1) == "IMM" else src,
                                                  shape).astype(np.float32)
                continue
            m = re.fullmatch(r"([AB]|S\d)2([AB]|S\d)", name)
            if m:
                reg[m.group(2)] = get(m.group(1)).copy()
                continue
            if name in ("EXP", "TANH", "SIGMOID", "RELU", "GELU", "GELU_BF", "SQUARE", "SQRT",
                        "RECIP", "NEG"):
                reg["A"] = _unary(name, get("A"))
                continue
            if name.endswith("_B") and name[:-2] in ("EXP", "TANH", "RELU", "SQUARE", "NEG"):
                reg["A"] = _unary(name[:-2], get("B"))
                continue
            if name.endswith("_IB") and name[:-3] in _XOPS:
                reg["A"] = np.broadcast_to(_xop(name[:-3], get("B"), np.float32(imm)), shape).astype(np.float32)
                continue
            if name in _XOPS:
                reg["A"] = _xop(name, get("A"), get("B"))
                continue
            m = re.fullmatch(r"(\w+)_([CRI])", name)
            if m and m.group(1) in _XOPS:
                x = np.float32(imm) if m.group(2) == "I" else lds(m.group(2), arg)
                reg["A"] = np.broadcast_to(_xop(m.group(1), get("A"), x), shape).astype(np.float32)
                continue
            if name in ("ST_F32", "ST_BF16"):
                idx = self._index(phase, arg)
                self._store(arg, idx, np.broadcast_to(get("A"), shape))
                continue
            if name == "ST_LDS":
                (self.col_lds if phase == "col" else self.row_lds)[arg] = get("A").copy()
                if phase == "elem":
                    raise AssertionError("an element program stores to LDS")
                continue
            if name in ("LDG_F32_A", "LDG_BF16_A"):
                reg["A"] = self._flat(arg)[self._addressed(arg)]
                continue
            if name in ("LDC_F32_A", "LDC_BF16_A"):
                sa, sb, split = arg & 0xFF, arg >> 8, int(imm)
                c = np.arange(self.C).reshape(1, -1)
                left = self._flat(sa)[np.where(c < split, self._addressed(sa), 0)]
                right = self._flat(sb)[np.where(c < split, 0, self._addressed(sb, split))]
                v = np.where(c < split, left, right)
                reg["A"] = np.broadcast_to(v, shape).astype(np.float32)
                continue
            if name == "LDT_A":
                s = self.code["transposed_slot"]
                assert s >= 0 and self.rs[s] == 1, "a staged transpose reads rows of its source"
                reg["A"] = self._flat(s)[self._addressed(s)]
                continue
            if name in ("RED", "RED_MAX", "RED_MV", "RED_SE"):
                assert phase == "elem", "a reduction outside the element phase"
                acc.append((name, get("A").astype(np.float64)))
                continue
            raise AssertionError(f"form {name} not replayed")

    def reduce(self, stage: dict, acc: list) -> None:
        kind = stage["reduce"]
        if kind == 0:
            assert not acc, "a stage without a reduction folds values"
            return
        names = {a for a, _ in acc}
        want = {1: {"RED"}, 2: {"RED"}, 3: {"RED_MAX"}, 4: {"RED_MV"}, 5: {"RED_SE"}}[kind]
        assert names == want, f"reduction {kind} folds {sorted(names)}"
        vals = [v for _, v in acc]
        with np.errstate(all="ignore"):
            if kind in (1, 2):
                assert len(vals) >= 1
                first = sum(v.sum(axis=1, keepdims=True) for v in vals)
                if kind == 2:
                    first = first / self.C
                second = None
            else:
                assert len(vals) == 1, "a max or paired reduction folds one value"
                x = vals[0]
                if kind == 3:
                    first, second = x.max(axis=1, keepdims=True), None
                elif kind == 4:
                    first = x.mean(axis=1, keepdims=True)
                    second = ((x - first) ** 2).mean(axis=1, keepdims=True)
                else:
                    first = x.max(axis=1, keepdims=True)
                    ms = np.where(first == -np.inf, 0.0, first)
                    second = np.exp(x - ms).sum(axis=1, keepdims=True)
        for v, lds_slot, ext in ((first, stage["reduce_lds"], stage["reduce_slot"]),
                                 (second, stage["reduce2_lds"], stage["reduce2_slot"])):
            if v is None:
                continue
            v = v.astype(np.float32)
            if lds_slot >= 0:
                self.row_lds[lds_slot] = v
            if ext >= 0:
                self._store(ext, self._index("row", ext), v)

    def replay(self) -> None:
        self.run(0, self.code["n_col"], "col", [])
        for st in self.code["stages"]:
            self.run(st["row_off"], st["row_len"], "row", [])
            acc: list = []
            self.run(st["elem_off"], st["elem_len"], "elem", acc)
            self.reduce(st, acc)


def replay_plan(graph, plan, inputs: Dict[int, np.ndarray]) -> Dict[int, np.ndarray]:
    """Every materialised tensor after the plan's groups ran in order, in its
    stored form (bf16 as uint16 bits).  Outputs start as NaN (bf16: a quiet
    NaN pattern) so a value no program stores shows."""
    mem: Dict[int, np.ndarray] = {}
    for t in plan.materialized():
        d = graph.tensors[t]
        shape = tuple(int(x) for x in d.shape)
        if d.role == "in":
            mem[t] = np.array(inputs[t]).reshape(shape)
        elif d.dtype == "bf16":
            mem[t] = np.full(shape, 0x7FC1, dtype=np.uint16)
        else:
            mem[t] = np.full(shape, np.nan, dtype=np.float32)
    for g in range(plan.num_groups):
        _Group(graph, plan, g, mem).replay()
    return mem
