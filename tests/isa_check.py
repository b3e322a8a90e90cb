"""Checks on the gfx950 assembly that hipcc emits for the kernels.

Two properties that the kernels rely on and that no GPU test shows reliably:

* No loop that holds a block barrier (s_barrier) leaves through an exec mask
  (s_andn2_b64 exec, exec, ... then s_cbranch_exec*).  Such a loop can keep
  some lanes of a wave iterating, and passing barriers, while the wave's other
  lanes wait outside it.  A block whose control code ran on one lane (thread
  0) inside its main loop was compiled that way and never finished.
* A k loop of a GEMM body (MFMAs fed by LDS DMA) waits on the vector-memory
  counter only for its ring: at most two such waits per iteration.  The
  compiler adds a full wait (vmcnt(0)) before LDS reads that it cannot tell
  apart from a DMA's target, which drains the ring at every k substep.

Loops are taken from the compiler's block comments ("Loop Header" /
"in Loop: Header=...").
"""
import os
import re
import subprocess

HIPCC = "/opt/rocm/bin/hipcc"
CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "sparse_moe_layer_fp32_amd", "csrc")
INCLUDE = os.path.join(os.path.dirname(CSRC), "..", "include")


def compile_asm(source, out_path):
    """gfx950 device assembly of one csrc file."""
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.normpath(INCLUDE), "-I", CSRC, "-S",
           "--offload-device-only", os.path.join(CSRC, source), "-o", out_path]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out_path).read()


def kernels(asm):
    """{kernel symbol: list of its lines} for every kernel in the file."""
    lines = asm.split("\n")
    out = {}
    for i, line in enumerate(lines):
        m = re.match(r"^(_Z\w+):", line)
        if not m or ".amdhsa" in line:
            continue
        j = i + 1
        while j < len(lines) and not re.match(r"^\s*s_endpgm", lines[j]):
            j += 1
        out[m.group(1)] = lines[i:j + 1]
    return out


def loops(body):
    """{header block: dict(parent, instrs)} with the instructions of the
    blocks whose innermost loop it is."""
    info = {}
    cur = None
    label_re = re.compile(r"^\.LBB(\d+_\d+):")
    for k, line in enumerate(body):
        s = line.strip()
        m = label_re.match(s)
        if m:
            name = "BB" + m.group(1)
            # the block's own comment and the comment lines after it
            com = s
            j = k + 1
            while j < len(body) and body[j].strip().startswith(";"):
                com += " " + body[j].strip()
                j += 1
            if "This Loop Header" in com or "This Inner Loop Header" in com:
                parent = re.search(r"Parent Loop (BB\d+_\d+)", com)
                info.setdefault(name, dict(parent=None, instrs=[]))
                # the innermost parent is the last "Parent Loop" named
                parents = re.findall(r"Parent Loop (BB\d+_\d+)", com)
                info[name]["parent"] = parents[-1] if parents else None
                cur = name
            else:
                h = re.search(r"in Loop: Header=(BB\d+_\d+)", com)
                cur = h.group(1) if h else None
                if cur:
                    info.setdefault(cur, dict(parent=None, instrs=[]))
            continue
        if re.match(r"^; %bb\.\d+:", s):
            h = re.search(r"in Loop: Header=(BB\d+_\d+)", s)
            cur = h.group(1) if h else None
            if cur:
                info.setdefault(cur, dict(parent=None, instrs=[]))
            continue
        if cur and s and not s.startswith(";") and not s.startswith("."):
            info[cur]["instrs"].append(s)
    return info


def _with_children(info):
    """Instructions of each loop including its nested loops."""
    total = {h: list(d["instrs"]) for h, d in info.items()}
    for h, d in info.items():
        p = d["parent"]
        seen = set()
        while p and p in total and p not in seen:
            seen.add(p)
            total[p].extend(d["instrs"])
            p = info[p]["parent"]
    return total


def barrier_loops_with_exec_exits(body):
    """Loops that hold an s_barrier (themselves or nested) and leave through
    an exec mask."""
    info = loops(body)
    total = _with_children(info)
    bad = []
    for h, d in info.items():
        ins = d["instrs"]
        exec_exit = any(a.startswith("s_andn2_b64 exec, exec,") and b.startswith("s_cbranch_exec")
                        for a, b in zip(ins, ins[1:]))
        if exec_exit and any(x.startswith("s_barrier") for x in total[h]):
            bad.append(h)
    return bad


def gemm_loop_vm_waits(body):
    """{header: vector-memory waits per iteration} of the innermost loops
    that issue LDS DMA and MFMAs."""
    out = {}
    for h, d in loops(body).items():
        ins = d["instrs"]
        if any(x.startswith("global_load_lds") for x in ins) and \
                sum(x.startswith("v_mfma") for x in ins) >= 4:
            out[h] = sum(1 for x in ins if x.startswith("s_waitcnt") and "vmcnt" in x)
    return out
