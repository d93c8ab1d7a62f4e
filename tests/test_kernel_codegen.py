"""Code-generation checks on the gfx950 assembly of the hot kernels (CPU only: hipcc cross-compiles).

The decode split kernel streams pages through rotating register sets; two silent compiler
outcomes defeat that without changing any result:
  * private-memory traffic (register spills, or a small array the compiler could not keep in
    registers): every scratch access is a vector-memory operation, and waiting on it waits on
    the page prefetch issued before it;
  * a full `s_waitcnt vmcnt(0)` inside the page loop, which drains the prefetch every page.
Both were seen once (a spilled 64-bit address and an lvalue conditional over an array) and cost
about 7 % of the kernel's time; these tests keep them out.
"""
import os
import re
import shutil
import subprocess

import pytest

from decode_attention_write_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")


def _assemble(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = B.COMMON + B.SOURCES[src] + ["-x", "hip", "--cuda-device-only", "-S",
                                       os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text().split("\n")


def _kernel_meta(lines):
    """Per kernel symbol: the fields of its entry in the code-object metadata."""
    meta, cur = {}, None
    for ln in lines:
        m = re.match(r"\s+\.name:\s+(\S+)", ln)
        if m:
            cur = m.group(1)
            meta[cur] = {}
            continue
        m = re.match(r"\s+\.(\w+):\s+(\S+)$", ln)
        if cur and m:
            meta[cur][m.group(1)] = m.group(2)
    return meta


def _page_loops(lines, symbol):
    """Bodies of the kernel's innermost loops that stream INT2 pages: wide global loads feeding
    matrix-core instructions (the BF16 sink/window loops use no matrix cores and wait per batch).
    A loop is its header block plus every block the compiler annotates as inside it (nested
    loops carry their annotation on the comment lines after the label)."""
    start = next(i for i, ln in enumerate(lines) if ln.startswith(symbol + ":"))
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    blocks, cur = [], None
    for ln in lines[start:end]:
        # named (.LBB) and unnamed (; %bb.N) basic blocks each start a block
        if re.match(r"^\.LBB\d+_\d+:", ln) or re.match(r"^; %bb\.\d+:", ln):
            cur = [ln]
            blocks.append(cur)
        elif cur is not None:
            cur.append(ln)
    def head(b):
        # the label line and the comment-only lines after it carry the loop annotations
        out = [b[0]]
        for ln in b[1:]:
            if not re.match(r"^\s+;", ln):
                break
            out.append(ln)
        return " ".join(out)

    def label(b):
        return b[0].split(":")[0][2:]  # .LBBx_y -> BBx_y

    heads = [head(b) for b in blocks]
    loops = {}
    for b, h in zip(blocks, heads):
        m = re.search(r"Loop Header: Depth=(\d+)", h)
        if not m:
            continue
        name, depth = label(b), m.group(1)
        members = [x for x, hx in zip(blocks, heads)
                   if x is b or f"Header={name} Depth={depth}" in hx or f"Parent Loop {name} Depth={depth}" in hx]
        body = [ln for x in members for ln in x]
        if any("global_load_dwordx4" in ln for ln in body) and any("v_mfma" in ln for ln in body):
            loops[name] = (members, body)
    # innermost: no other streaming loop's header among its blocks
    return [body for name, (members, body) in loops.items()
            if not any(label(x) in loops and label(x) != name for x in members)]


def test_decode_split_kernel_codegen(tmp_path):
    lines = _assemble("decode_mfma.hip", tmp_path)
    meta = _kernel_meta(lines)
    kernels = [k for k in meta if "k_decode_mfma" in k]
    assert len(kernels) == 4, kernels  # GQA 1, 2, 4, 8
    for k in kernels:
        assert meta[k]["vgpr_spill_count"] == "0", (k, meta[k])
        assert meta[k]["private_segment_fixed_size"] == "0", (k, meta[k])
        loops = _page_loops(lines, k)
        assert loops, k
        for body in loops:
            assert not any("scratch_" in b for b in body), k
            assert not any(re.search(r"s_waitcnt\s+vmcnt\(0\)", b) for b in body), k


def test_write_kernel_no_private_memory(tmp_path):
    meta = _kernel_meta(_assemble("write.hip", tmp_path))
    for k, m in meta.items():
        assert m["vgpr_spill_count"] == "0", (k, m)
        assert m["private_segment_fixed_size"] == "0", (k, m)
