"""Build check of an MFMA hazard that inline asm hides from the compiler.

An MFMA that reads a vector register (VGPR or AGPR) written by a VALU
instruction needs two wait states between the two (CDNA3/CDNA4 ISA, required
wait states for matrix instructions).  The attend kernels issue their MFMAs
from inline asm, mostly without nops, because their operands arrive from LDS
or global loads, which the waitcnt counters cover.  The compiler cannot see
that the asm is an MFMA, so nothing stops it from placing, say, a register
copy right before one.  This check compiles the device code to assembly with
the library's flags and verifies, for every v_mfma, that no VALU instruction
writing one of its source registers lies within the two wait states before
it, along any path into it (predecessor blocks included).  It fails the build
otherwise.
"""
from __future__ import annotations

import re
import subprocess
import sys
from typing import Dict, List, Set, Tuple

_REG = re.compile(r"\b([va])(?:(\d+)|\[(\d+):(\d+)\])")
_LABEL = re.compile(r"^(\.LBB\d+_\d+|[A-Za-z_][\w.$]*):")
_NEED = 2  # wait states between a VALU write and an MFMA read


def _regs(op: str) -> Set[Tuple[str, int]]:
    out = set()
    for m in _REG.finditer(op):
        kind = m.group(1)
        if m.group(2) is not None:
            out.add((kind, int(m.group(2))))
        else:
            out.update((kind, r) for r in range(int(m.group(3)), int(m.group(4)) + 1))
    return out


def _split_ops(rest: str) -> List[str]:
    ops, depth, cur = [], 0, ""
    for ch in rest:
        if ch == "[":
            depth += 1
        elif ch == "]":
            depth -= 1
        if ch == "," and depth == 0:
            ops.append(cur.strip())
            cur = ""
        else:
            cur += ch
    if cur.strip():
        ops.append(cur.strip())
    return ops


def _valu_dst(mn: str, ops: List[str]) -> Set[Tuple[str, int]]:
    """Vector registers written by a VALU instruction (empty for other kinds)."""
    if not mn.startswith("v_") or mn.startswith(("v_mfma", "v_cmp", "v_readlane", "v_readfirstlane")):
        return set()
    if not ops:
        return set()
    return _regs(ops[0])


def _wait_states(mn: str, ops: List[str]) -> int:
    if mn == "s_nop":
        return int(ops[0], 0) + 1 if ops else 1
    return 1


class _Fn:
    def __init__(self, name: str):
        self.name = name
        self.blocks: List[Tuple[str, List[Tuple[str, List[str], str]]]] = []


def _parse(asm: str) -> List[_Fn]:
    fns: List[_Fn] = []
    fn = None
    for raw in asm.split("\n"):
        line = raw.split(";")[0].rstrip()
        s = line.strip()
        if not s:
            continue
        m = _LABEL.match(s)
        if m:
            name = m.group(1)
            if not name.startswith(".L"):
                if name.startswith("_Z") or "kernel" in name:
                    fn = _Fn(name)
                    fns.append(fn)
                    fn.blocks.append((name, []))
                continue
            if fn is not None:
                fn.blocks.append((name, []))
            continue
        if s.startswith("."):
            continue
        if fn is None:
            continue
        parts = s.split(None, 1)
        mn = parts[0]
        ops = _split_ops(parts[1]) if len(parts) > 1 else []
        fn.blocks[-1][1].append((mn, ops, s))
        if mn == "s_endpgm":
            fn = None
    return fns


def _preds(fn: _Fn) -> Dict[int, List[Tuple[int, int]]]:
    """For each block, (predecessor block, index of its last instruction on that edge)."""
    index = {name: i for i, (name, _) in enumerate(fn.blocks)}
    preds: Dict[int, List[Tuple[int, int]]] = {i: [] for i in range(len(fn.blocks))}
    for i, (_, ins) in enumerate(fn.blocks):
        falls = True
        for k, (mn, ops, _) in enumerate(ins):
            if mn.startswith("s_cbranch") or mn == "s_branch":
                tgt = ops[0] if ops else ""
                if tgt in index:
                    preds[index[tgt]].append((i, k))
                if mn == "s_branch":
                    falls = False
            if mn in ("s_endpgm", "s_setpc_b64"):
                falls = False
        if falls and i + 1 < len(fn.blocks):
            preds[i + 1].append((i, len(ins) - 1))
    return preds


def _scan_back(fn, preds, blk, pos, srcs, have, seen) -> List[str]:
    """Instructions writing `srcs` within the wait states still missing."""
    bad = []
    ins = fn.blocks[blk][1]
    k = pos
    while k >= 0:
        mn, ops, text = ins[k]
        if _valu_dst(mn, ops) & srcs:
            bad.append(text)
        have += _wait_states(mn, ops)
        if have >= _NEED:
            return bad
        k -= 1
    for p, last in preds[blk]:
        key = (p, last, have)
        if key in seen:
            continue
        seen.add(key)
        bad += _scan_back(fn, preds, p, last, srcs, have, seen)
    return bad


def check_asm(asm: str) -> List[str]:
    """Violations as readable strings (empty when the code is clean)."""
    problems = []
    for fn in _parse(asm):
        preds = _preds(fn)
        for b, (label, ins) in enumerate(fn.blocks):
            for k, (mn, ops, text) in enumerate(ins):
                if not mn.startswith("v_mfma"):
                    continue
                srcs = set()
                for op in ops[1:4]:
                    srcs |= _regs(op)
                bad = _scan_back(fn, preds, b, k - 1, srcs, 0, set())
                for w in bad:
                    problems.append(f"{fn.name} {label}: '{w}' feeds '{text}' without two wait states")
    return problems


def device_asm(src: str, hipcc: str, flags: List[str]) -> str:
    """Device assembly of `src` for gfx950 with the library's compile flags."""
    keep = [f for f in flags if f not in ("-shared", "-fPIC")]
    cmd = [hipcc, *keep, "-S", "--offload-device-only", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"device assembly failed ({r.returncode}):\n{r.stderr[-3000:]}")
    return r.stdout


def check_source(src: str, hipcc: str, flags: List[str]) -> List[str]:
    return check_asm(device_asm(src, hipcc, flags))


if __name__ == "__main__":
    from mla_latent_cache_absorbed_amd import build as _b
    probs = check_source(_b.SRC, _b.HIPCC, _b.FLAGS)
    for p in probs:
        print(p)
    print(f"{len(probs)} MFMA operand hazards")
    sys.exit(1 if probs else 0)
