"""Static check of the loads the compiler does not track.

A few kernels load metadata or operand fragments with inline-assembly global
loads (load_untracked / load_untracked_x4 in csrc/common.h): the compiler adds
no wait for them, so the code waits explicitly with s_waitcnt before using the
value.  Nothing stops the register allocator from touching the destination
registers before that wait (a copy of them once staged stale values), so this
test compiles the kernels to AMD assembly, here, and checks every such load on
every control-flow path: until an s_waitcnt vmcnt(N) with N no larger than the
vector-memory instructions issued since the load (vmcnt counts them in issue
order, so the load has then completed), no instruction may read or write any of
its destination registers.

The walk follows branches (both ways for conditional ones, except that a
branch on vcc, scc or exec whose value the path has already branched on, with
no write to it since, goes the one way that value allows) and stops a path at
the covering wait; a path that reaches the end of the kernel, or loops back to
a state already explored, is fine.  Register operands are parsed from the
operand text (v12, v[12:15]).

The same assembly also pins the stores inside the attention's key-tile loop,
which its explicit wait counts allow for.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_kv_amd", "csrc")
SOURCES = ("qkv_rope_cachewrite.hip", "sched_attention.hip")
VMEM = ("global_", "buffer_", "scratch_", "flat_")
REG = re.compile(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]")
VMCNT = re.compile(r"vmcnt\((\d+)\)")


def _assemble(src: str) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = os.path.join("/tmp", f"untracked_{os.getpid()}_{os.path.basename(src)}.s")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        text = f.read()
    os.remove(out)
    return text


def _regs(operands: str) -> set:
    s = set()
    for m in REG.finditer(operands):
        if m.group(1) is not None:
            s.add(int(m.group(1)))
        else:
            s.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return s


def _functions(text: str):
    """(name, [instruction lines]) per kernel; labels kept as 'LABEL:'."""
    funcs = []
    cur = None
    for raw in text.split("\n"):
        line = raw.split(";")[0].rstrip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        m = re.match(r"^(_Z\S+):", raw)
        if m:
            cur = (m.group(1), [])
            funcs.append(cur)
            continue
        if cur is None:
            continue
        s = line.strip()
        if s.startswith(".Lfunc_end"):
            cur = None
            continue
        if not s or s.startswith("."):
            if re.match(r"^\.LBB\w+:", s):
                cur[1].append(s)
            continue
        cur[1].append(s)
    return funcs


# scalar instructions that leave SCC alone (every other s_ instruction is taken to write it)
_SCC_KEEP = ("s_cbranch", "s_branch", "s_waitcnt", "s_nop", "s_barrier", "s_mov_b32", "s_mov_b64", "s_movk",
             "s_load", "s_buffer_load", "s_setprio", "s_sleep", "s_endpgm", "s_getpc", "s_sendmsg")
# branch -> (condition register, value it has when the branch is taken)
_BRANCH = {"s_cbranch_vccz": ("vcc", 0), "s_cbranch_vccnz": ("vcc", 1), "s_cbranch_scc0": ("scc", 0),
           "s_cbranch_scc1": ("scc", 1), "s_cbranch_execz": ("exec", 0), "s_cbranch_execnz": ("exec", 1)}


def _written_conditions(op: str, args: str) -> set:
    """Condition registers (vcc, scc, exec) an instruction may change."""
    if op.startswith("s_cbranch"):
        return set()
    out = set()
    if "vcc" in args:
        out.add("vcc")
    if "exec" in args:
        out.add("exec")
    if op.startswith("s_") and not op.startswith(_SCC_KEEP):
        out.add("scc")
    return out


def _check(name: str, code: list) -> list:
    labels = {l[:-1]: i for i, l in enumerate(code) if l.endswith(":") and l.startswith(".LBB")}
    problems = []
    in_asm = False
    loads = []
    for i, l in enumerate(code):
        if l.startswith(";;#ASMSTART"):
            in_asm = True
        elif l.startswith(";;#ASMEND"):
            in_asm = False
        elif in_asm and l.startswith("global_load") and "_lds" not in l:
            parts = l.split(None, 1)
            dest = _regs(parts[1].split(",")[0])
            loads.append((i, dest))
    for i0, dest in loads:
        # a path state is (instruction, VMEM instructions since the load, the
        # condition registers whose value this path has branched on and not
        # changed since): branches on a known value follow one way only
        seen = set()
        stack = [(i0 + 1, 0, frozenset())]
        while stack:
            i, n, known = stack.pop()
            while i < len(code):
                if (i, n, known) in seen:
                    break
                seen.add((i, n, known))
                l = code[i]
                if l.endswith(":") or l.startswith(";;#ASM"):
                    i += 1
                    continue
                op = l.split(None, 1)[0]
                args = l.split(None, 1)[1] if " " in l else ""
                if op == "s_waitcnt":
                    m = VMCNT.search(args)
                    if m and int(m.group(1)) <= n:
                        break                               # the load has completed on this path
                    i += 1
                    continue
                if op == "s_endpgm":
                    break
                if _regs(args) & dest:
                    problems.append(f"{name}: line {i} touches {sorted(dest)} before the wait for the "
                                    f"load at line {i0}: {l}")
                    break
                if op.startswith(VMEM):
                    n = min(n + 1, 64)
                wr = _written_conditions(op, args)
                if wr:
                    known = frozenset(kv for kv in known if kv[0] not in wr)
                if op == "s_branch":
                    i = labels[args.strip()]
                    continue
                if op in _BRANCH:
                    reg, taken_val = _BRANCH[op]
                    val = dict(known).get(reg)
                    target = labels[args.strip()]
                    if val is None:
                        stack.append((target, n, known | {(reg, taken_val)}))
                        known = known | {(reg, 1 - taken_val)}
                    elif val == taken_val:
                        i = target
                        continue
                elif op.startswith("s_cbranch"):
                    stack.append((labels[args.strip()], n, known))
                i += 1
    return problems, len(loads)


@pytest.fixture(scope="module")
def assembly():
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(_assemble, SOURCES)))


def test_untracked_loads_are_waited_for_before_any_use(assembly):
    total = 0
    problems = []
    for src, text in assembly.items():
        for name, code in _functions(text):
            p, n = _check(name, code)
            problems += p
            total += n
    assert total > 0, "no untracked loads found: the check would pass vacuously"
    assert not problems, "\n".join(problems[:20])


def _main_loop(code: list):
    """The longest backward-branch range that contains MFMAs (the key-tile loop)."""
    labels = {l[:-1]: i for i, l in enumerate(code) if l.endswith(":") and l.startswith(".LBB")}
    best = None
    for i, l in enumerate(code):
        parts = l.split(None, 1)
        if parts and (parts[0].startswith("s_cbranch") or parts[0] == "s_branch") and len(parts) > 1:
            a = labels.get(parts[1].strip())
            if a is not None and a < i and any("v_mfma" in x for x in code[a:i]):
                if best is None or i - a > best[1] - best[0]:
                    best = (a, i)
    return code[best[0]:best[1]] if best else []


def test_attention_loop_stores_match_its_wait_counts(assembly):
    """The attention's stage waits let the stores of the window rows'
    probabilities stay in flight: three per row tile per key tile (two
    16-byte stores and the exponent reference).  Vector-memory stores share
    the counter with the copies, so fewer stores in the loop than the waits
    allow for would let a wait return before its tile's copies have landed:
    every attention kernel's key-tile loop must hold exactly 3 x RT stores."""
    seen = 0
    for name, code in _functions(assembly["sched_attention.hip"]):
        m = re.search(r"attn_bf16_kernelILi(\d+)ELi(\d+)", name)
        if not m:
            continue
        rt = int(m.group(1))
        loop = _main_loop(code)
        stores = [l for l in loop if l.split(None, 1)[0].startswith(("global_store", "buffer_store", "flat_store"))]
        assert len(stores) == 3 * rt, (name, stores)
        seen += 1
    assert seen >= 6, "attention kernels not found"


def test_the_checker_flags_a_use_before_the_wait():
    # a hand-written sequence: the destination is copied before the covering
    # wait (flagged), and the same copy after it (not flagged); a branch
    # around the wait is followed both ways
    bad = [";;#ASMSTART", "global_load_dword v5, v[2:3], off", ";;#ASMEND",
           "global_load_lds_dwordx4 v[8:9], off", "v_mov_b32_e32 v7, v5", "s_waitcnt vmcnt(1)", "s_endpgm"]
    good = [";;#ASMSTART", "global_load_dwordx4 v[4:7], v[2:3], off", ";;#ASMEND",
            "global_load_lds_dwordx4 v[8:9], off", "s_waitcnt vmcnt(1)", "v_mov_b32_e32 v10, v6", "s_endpgm"]
    branchy = [";;#ASMSTART", "global_load_dword v5, v[2:3], off", ";;#ASMEND",
               "s_cbranch_scc1 .LBB0_2", "s_waitcnt vmcnt(0)", ".LBB0_2:", "v_add_u32_e32 v6, v5, v5", "s_endpgm"]
    # an if / else compiled as two branches on the same vcc: each side issues
    # one copy, so the wait for one covers the load on both real paths; the
    # walk must not take "skip both" (vcc unchanged between the branches) ...
    diamond = [";;#ASMSTART", "global_load_dword v5, v[2:3], off", ";;#ASMEND",
               "s_cbranch_vccz .LBB0_1", "global_load_lds_dwordx4 v[8:9], off", ".LBB0_1:",
               "s_cbranch_vccnz .LBB0_2", "global_load_lds_dwordx4 v[8:9], off nt", ".LBB0_2:",
               "s_waitcnt vmcnt(1)", "v_add_u32_e32 v6, v5, v5", "s_endpgm"]
    # ... unless vcc changes in between, on the path that skipped the first copy
    rewritten = diamond[:6] + ["v_cmp_lt_i32_e32 vcc, 0, v7"] + diamond[6:]
    assert _check("bad", bad)[0]
    assert not _check("good", good)[0]
    assert _check("branchy", branchy)[0]
    assert not _check("diamond", diamond)[0]
    assert _check("rewritten", rewritten)[0]
