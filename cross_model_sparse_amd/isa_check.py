"""Static checks of the generated gfx950 code of the retrieval kernels.

The retrieval loop issues its vector-memory operations (direct-to-LDS copies
and their counter waits) through inline asm, where the compiler neither
inserts hazard wait states nor tracks outstanding loads.  These checks run on
`hipcc -S` output and guard the properties that inline asm makes the
programmer's job:

  scratch      no kernel spills to scratch memory;
  inflight     no instruction reads or writes a VGPR while it is the
               destination of a vector load that no `s_waitcnt vmcnt` has
               retired yet (loads retire in issue order; the walk follows the
               control-flow graph, takes uniform branches whose condition is a
               known constant, and assumes a full exec mask);
  valu_sgpr    no vector-memory instruction reads an SGPR fewer than 5 wait
               states after a VALU instruction wrote it (lane reads, compare
               masks, carry outs);
  m0_dma       no LDS DMA directly follows the SALU write of M0 it uses;
  m0_live      no instruction outside the copy statements reads M0 while the
               last M0 write before it (in program order) is a copy
               statement's: a value the compiler keeps in M0 must not be
               live across them.

    python -m cross_model_sparse_amd.isa_check [kernel.hip]
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from collections import deque
from pathlib import Path

HERE = Path(__file__).resolve().parent
VMEM = re.compile(r"(global|buffer|flat|scratch)_(load|store|atomic)")


def _vregs(tok: str) -> frozenset:
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def _sgpr_ranges(text: str):
    for m in re.finditer(r"s\[(\d+):(\d+)\]|\bs(\d+)\b", text):
        lo = int(m.group(1) or m.group(3))
        hi = int(m.group(2) or m.group(3))
        yield lo, hi


def _functions(lines):
    """name -> list of (line number, instruction text) of each kernel body."""
    out = {}
    cur = None
    for ln, raw in enumerate(lines, 1):
        if re.match(r"^_Z\S+:", raw):
            cur = raw.split(":")[0]
            out[cur] = []
            continue
        if cur is None:
            continue
        if raw.startswith(".Lfunc_end"):
            cur = None
            continue
        s = raw.split(";")[0].strip()
        if s:
            out[cur].append((ln, s))
    return out


def _metadata(lines):
    meta, cur = {}, None
    for raw in lines:
        m = re.match(r"\s+\.name:\s+(\S+)", raw)
        if m:
            cur = m.group(1)
            meta.setdefault(cur, {})
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_count):\s+(\d+)", raw)
        if m and cur:
            meta[cur][m.group(1)] = int(m.group(2))
    return meta


def _blocks(body):
    order, blocks, succ = [], {}, {}
    cur = "@0"
    order.append(cur)
    blocks[cur] = []
    n = 0
    for ln, s in body:
        if re.match(r"^\.LBB\S+:$", s):
            cur = s[:-1]
            order.append(cur)
            blocks[cur] = []
            continue
        if s.startswith("."):
            continue
        blocks[cur].append((ln, s))
        op = s.split()[0]
        if op.startswith("s_cbranch") or op in ("s_branch", "s_endpgm"):
            n += 1
            cur = f"@{n}"
            order.append(cur)
            blocks[cur] = []
    for k, b in enumerate(order):
        last = blocks[b][-1][1] if blocks[b] else ""
        op = last.split()[0] if last else ""
        nxt = order[k + 1] if k + 1 < len(order) else None
        if op == "s_branch":
            succ[b] = [last.split()[1]]
        elif op == "s_cbranch_execz":        # full exec mask: never taken
            succ[b] = [nxt] if nxt else []
        elif op == "s_cbranch_execnz":       # full exec mask: always taken
            succ[b] = [last.split()[1]]
        elif op.startswith("s_cbranch"):
            succ[b] = [last.split()[1]] + ([nxt] if nxt else [])
        elif op == "s_endpgm":
            succ[b] = []
        else:
            succ[b] = [nxt] if nxt else []
    return order, blocks, succ


_WAIT_VM = re.compile(r"s_waitcnt\s+.*vmcnt\((\d+)\)")


def _decode(s):
    """One instruction as the walk in _inflight needs it."""
    parts = s.replace(",", " ").split()
    op, ops = parts[0], parts[1:]
    salu = None
    if op.startswith("s_") and ops:
        dst = ops[0]
        if op == "s_mov_b64" and len(ops) > 1 and ops[1] in ("-1", "0"):
            salu = ("set", dst, int(ops[1]))
        elif op == "s_andn2_b64" and dst == "vcc" and len(ops) > 2 and ops[1] == "exec":
            salu = ("andn2", ops[2])
        else:
            rng = set(range(*map(int, dst[2:-1].split(":")))) if dst.startswith("s[") else None
            salu = ("kill", dst, rng)
    m = _WAIT_VM.match(s)
    if m:
        return (salu, "wait", int(m.group(1)), None)
    if VMEM.match(op):
        is_load = "load" in op
        dest = _vregs(ops[0]) if is_load and "lds" not in op else frozenset()
        srcs = ops[1:] if is_load else ops
        src = frozenset().union(*[_vregs(t) for t in srcs]) if srcs else frozenset()
        return (salu, "vmem", dest, src)
    if op.startswith("v_") or op.startswith("ds_"):
        regs = frozenset().union(*[_vregs(t) for t in ops]) if ops else frozenset()
        return (salu, "use", regs, None)
    return (salu, None, None, None)


def _inflight(body, max_states=64):
    """Lines touching the destination VGPRs of outstanding vector loads.

    The walk follows every path of the kernel's control-flow graph (scalar
    branches on a known vcc are resolved) to a fixed point.  A state holds,
    for each outstanding load that writes VGPRs, its registers and how many
    vector-memory operations were issued after it (capped at 64: any
    vmcnt(n) retires such a load, as n <= 63); loads into LDS only add to
    those counts.  That is exactly what `s_waitcnt vmcnt(n)` needs (it
    retires every load with n or more operations issued after it), and it
    keeps the number of states small where copies of varying count are in
    flight."""
    order, blocks, succ = _blocks(body)
    code = {b: [(ln, s, _decode(s)) for ln, s in blocks[b]] for b in order}
    states = {b: set() for b in order}
    states["@0"].add(((), frozenset()))
    work = deque(["@0"])
    bad = {}
    while work:
        b = work.popleft()
        for fifo0, consts0 in list(states[b]):
            fifo, consts = list(fifo0), dict(consts0)
            for ln, s, (salu, kind, x, y) in code[b]:
                if salu is not None:
                    if salu[0] == "set":
                        consts[salu[1]] = salu[2]
                    elif salu[0] == "andn2" and salu[1] in consts:
                        consts["vcc"] = 1 if consts[salu[1]] == 0 else 0
                    elif consts:
                        dst, a = (salu[1], salu[2]) if salu[0] == "kill" else ("vcc", None)
                        for k in list(consts):
                            if k == dst:
                                consts.pop(k, None)
                            elif a is not None and k.startswith("s["):
                                if a & set(range(*map(int, k[2:-1].split(":")))):
                                    consts.pop(k, None)
                if kind == "wait":
                    fifo = [(d, n) for d, n in fifo if n < x]
                elif kind == "vmem":
                    for d, _ in fifo:
                        if y & d or x & d:
                            bad.setdefault(ln, s)
                    fifo = [(d, min(n + 1, 64)) for d, n in fifo]
                    if x:
                        fifo.append((x, 0))
                elif kind == "use" and fifo:
                    for d, _ in fifo:
                        if x & d:
                            bad.setdefault(ln, s)
            out = (tuple(fifo), frozenset(consts.items()))
            last = blocks[b][-1][1] if blocks[b] else ""
            nbs = succ[b]
            if last.startswith("s_cbranch_vccnz") and "vcc" in consts:
                nbs = nbs[:1] if consts["vcc"] else nbs[1:]
            elif last.startswith("s_cbranch_vccz") and "vcc" in consts:
                nbs = nbs[1:] if consts["vcc"] else nbs[:1]
            for nb in nbs:
                if nb in states and out not in states[nb]:
                    if len(states[nb]) < max_states:
                        states[nb].add(out)
                        work.append(nb)
                    elif blocks[nb]:
                        # a state left unexplored would make the walk unsound:
                        # report it rather than pass the kernel
                        ln0 = blocks[nb][0][0]
                        bad.setdefault(ln0, f"(walk incomplete: more than {max_states} states) "
                                            + blocks[nb][0][1])
    return sorted(bad.items())


# VALU instructions whose second operand is a scalar destination (carry out,
# division scale flag): the VOP3b forms.
_VOP3B = re.compile(r"^v_(add|sub|subrev|addc|subb|subbrev)_co_|^v_div_scale_|^v_mad_[iu]64_[iu]32")


def _sgprs(tok: str) -> frozenset:
    if tok == "vcc":
        return frozenset({106, 107})
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return frozenset(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return frozenset({int(m.group(1))}) if m else frozenset()


def _valu_sgpr_dests(s: str) -> frozenset:
    """SGPRs a VALU instruction writes: lane reads, compare masks, carries."""
    parts = s.replace(",", " ").split()
    op, ops = parts[0], parts[1:]
    if not op.startswith("v_") or not ops:
        return frozenset()
    if op.startswith(("v_readfirstlane", "v_readlane")) or (op.startswith("v_cmp") and not op.startswith("v_cmpx")):
        return _sgprs(ops[0])
    if _VOP3B.match(op) and len(ops) > 1:
        return _sgprs(ops[1])
    return frozenset()


def _linear_hazards(body):
    insts = [s for _, s in body if not s.startswith(".")]
    lines = [ln for ln, s in body if not s.startswith(".")]
    valu_sgpr, m0 = [], []
    for i, s in enumerate(insts):
        dst = _valu_sgpr_dests(s)
        if dst:
            ws = 0
            for j in range(i + 1, min(len(insts), i + 8)):
                x = insts[j]
                if VMEM.match(x.split()[0]) and ws < 5:
                    if any(n in dst for lo, hi in _sgpr_ranges(x) for n in range(lo, hi + 1)):
                        valu_sgpr.append((lines[j], x))
                k = re.match(r"s_nop (\d+)", x)
                ws += int(k.group(1)) + 1 if k else 1
        if s.startswith("s_mov_b32 m0") and i + 1 < len(insts):
            nxt = insts[i + 1]
            if "lds" in nxt and VMEM.match(nxt.split()[0]):
                m0.append((lines[i + 1], nxt))
    return valu_sgpr, m0


# Instructions that read M0 without naming it (gfx9 family): indexed register
# moves, GDS/ordered LDS operations, messages and LDS-direct loads.
_M0_IMPLICIT = re.compile(r"^(v_movrel|s_movrel|s_sendmsg|ds_gws|ds_ordered|ds_append|ds_consume|"
                          r"s_set_gpr_idx|v_interp|ds_read_addtid|ds_write_addtid)")


def _is_copy_m0(insts, i):
    """insts[i] is the M0 write of a copy statement: s_mov_b32 m0, sN, then
    s_nop 0, then the LDS DMA."""
    return (insts[i].startswith("s_mov_b32 m0,") and i + 2 < len(insts)
            and insts[i + 1].startswith("s_nop 0") and "lds" in insts[i + 2]
            and VMEM.match(insts[i + 2].split()[0]) is not None)


def _m0_live(body):
    """Lines that read M0 after a copy statement overwrote it (linear order)."""
    insts = [s for _, s in body if not s.startswith(".")]
    lines = [ln for ln, s in body if not s.startswith(".")]
    writer, bad = None, []
    i = 0
    while i < len(insts):
        s = insts[i]
        if _is_copy_m0(insts, i):
            writer = "copy"
            i += 3
            continue
        parts = s.replace(",", " ").split()
        op, ops = parts[0], parts[1:]
        reads = _M0_IMPLICIT.match(op) is not None or ("m0" in ops[1:]) or \
            (op.startswith("s_") and ops[:1] != ["m0"] and "m0" in ops)
        if ops[:1] == ["m0"] and not op.startswith(("v_", "ds_", "global_", "buffer_")):
            writer = "compiler"
        elif reads and writer == "copy":
            bad.append((lines[i], s))
        i += 1
    return bad


def check_asm(path: str, pattern: str = "k_retrieve_mfma"):
    """Findings per kernel whose name contains `pattern`: a dict kernel ->
    {'scratch': bytes, 'inflight': [...], 'valu_sgpr': [...], 'm0_dma': [...],
    'm0_live': [...]}."""
    lines = open(path).read().split("\n")
    meta = _metadata(lines)
    out = {}
    for name, body in _functions(lines).items():
        if pattern not in name:
            continue
        valu_sgpr, m0 = _linear_hazards(body)
        out[name] = {"scratch": meta.get(name, {}).get("private_segment_fixed_size", 0),
                     "vgpr": meta.get(name, {}).get("vgpr_count"),
                     "inflight": _inflight(body), "valu_sgpr": valu_sgpr, "m0_dma": m0,
                     "m0_live": _m0_live(body)}
    return out


def compile_to_asm(src: Path, out: Path) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", str(HERE / "csrc"), "-I", str(HERE.parent / "include"), "-o", str(out), str(src)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)


def main(argv):
    src = Path(argv[1]) if len(argv) > 1 else HERE / "csrc" / "k_retrieve.hip"
    with tempfile.TemporaryDirectory() as td:
        asm = Path(td) / "k.s"
        compile_to_asm(src, asm)
        res = check_asm(str(asm), pattern="k_")
    bad = 0
    for name, r in sorted(res.items()):
        n = (r["scratch"] + len(r["inflight"]) + len(r["valu_sgpr"]) + len(r["m0_dma"])
             + len(r["m0_live"]))
        bad += n
        print(f"{name[:60]:60s} vgpr {r['vgpr']} scratch {r['scratch']} inflight "
              f"{len(r['inflight'])} valu_sgpr {len(r['valu_sgpr'])} m0_dma {len(r['m0_dma'])} "
              f"m0_live {len(r['m0_live'])}")
    print(f"{len(res)} kernels, {bad} findings")
    return 1 if bad or not res else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
