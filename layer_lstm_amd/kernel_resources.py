"""Register use of the path's kernels, from the compiler's own reports.

    python -m layer_lstm_amd.kernel_resources [--out FILE] [--match NAME ...]

Compiles the kernel sources for gfx950 with the library's flags plus
-Rpass-analysis=kernel-resource-usage and -save-temps (device code only, in a
temporary folder; liblstm.so is not touched) and prints, for every kernel
instance whose demangled name contains one of the --match strings (default:
the instances the four workloads of layer_lstm_amd/synth.py launch):

  - VGPRs, AGPRs, SGPRs, SGPRs spilled (to VGPR lanes), VGPRs spilled and
    scratch bytes per lane, as the compiler reports them;
  - inside the kernel's step loop (the outermost loop with the most basic
    blocks), the instructions that move spilled values: v_readlane_b32 /
    v_writelane_b32 (SGPR spill reloads and stores) and scratch loads and
    stores (VGPR spills), split into blocks on the per-step path and blocks
    of the failure and stamp paths (those that hold a global atomic -- the
    error word -- or an s_memrealtime -- the phase stamps -- which run only
    when a wait times out or when stamps are requested).

The counts are static (instructions in the loop body, each block once); a
block on the per-step path may still sit behind a branch that a step does
not take.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import os
import re
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

from layer_lstm_amd import build as _build  # noqa: E402

SOURCES = ("recurrent.hip", "recurrent_bwd.hip", "recurrent_vec.hip", "gemm.hip")
# kernel instances of the four workloads (rocprofv3 names, profiles/kernels_*.txt)
DEFAULT_MATCH = (
    "fwd_rec_kernel<unsigned short, 2, 16, 0, 8, 2, false>",   # bf16_T256_B256_I1024_H1024
    "bwd_col_kernel<unsigned short, 2, 2, 16, 8, true>",
    "fwd_rec_kernel<unsigned short, 1, 16, 0, 8, 2, false>",   # bf16_T128_B64_I512_H1024
    "bwd_col_kernel<unsigned short, 1, 2, 16, 8, true>",
    "fwd_rec_kernel<unsigned short, 1, 16, 0, 8, 2, true>",    # bf16_T512_B16_I1024_H2048
    "bwd_col_kernel<unsigned short, 1, 1, 32, 8, false>",
    "fwd_vec_kernel<",                                          # f32_T64_B32_I256_H256
    "bwd_vec_kernel<",
    "gemm_lds_kernel<unsigned short",
    "gemm_lds_multi_kernel<unsigned short",
)
FIELDS = (("VGPRs", "vgpr"), ("AGPRs", "agpr"), ("TotalSGPRs", "sgpr"), ("SGPRs Spill", "sgpr_spill"),
          ("VGPRs Spill", "vgpr_spill"), ("ScratchSize [bytes/lane]", "scratch"))


def demangle(names):
    tool = None
    for cand in ("/opt/rocm/llvm/bin/llvm-cxxfilt", shutil.which("llvm-cxxfilt"), shutil.which("c++filt")):
        if cand and os.path.exists(cand):
            tool = cand
            break
    if tool is None:
        return {n: n for n in names}
    r = subprocess.run([tool], input="\n".join(names), capture_output=True, text=True)
    out = r.stdout.splitlines()
    return dict(zip(names, out)) if len(out) == len(names) else {n: n for n in names}


def compile_one(src: str, tmp: str):
    cc = _build.hipcc()
    wd = os.path.join(tmp, src.replace(".", "_"))
    os.makedirs(wd, exist_ok=True)
    cmd = [cc, *_build.flags(), "--offload-device-only", "-save-temps", "-Rpass-analysis=kernel-resource-usage",
           "-c", os.path.join(_build.CSRC, src), "-o", os.path.join(wd, "out.o")]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=wd)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    asm = [os.path.join(wd, f) for f in os.listdir(wd) if f.endswith(".s") and "amdgcn" in f]
    return src, r.stderr, asm[0] if asm else None


def parse_remarks(text: str):
    rows, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = rows.setdefault(m.group(1), {})
            continue
        if cur is None:
            continue
        for key, name in FIELDS:
            m = re.search(r"\s" + re.escape(key) + r": (\d+)", line)
            if m:
                cur[name] = int(m.group(1))
    return rows


def loop_moves(asm_text: str, fn: str):
    """Spill moves inside the step loop of function fn (the outermost loop
    with the most basic blocks, its nested loops included): (path, off-path)
    counts of v_readlane_b32, v_writelane_b32 and scratch instructions."""
    start = asm_text.find("\n" + fn + ":")
    end = asm_text.find(".Lfunc_end", start)
    if start < 0 or end < 0:
        return None
    lines = asm_text[start:end].splitlines()
    blocks, cur = [], None
    children = {}   # loop header -> nested loop headers
    depth1 = set()
    for i, l in enumerate(lines):
        m = re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)(.*)", l)
        if m:
            own = m.group(1)[2:-1] if m.group(1).startswith(".L") else None
            note = l
            j = i + 1
            while j < len(lines) and lines[j].lstrip().startswith(";") and not re.match(r"^; %bb", lines[j]):
                note += "\n" + lines[j]
                j += 1
            hm = re.search(r"=>This (?:Inner )?Loop Header: Depth=(\d+)", note)
            if hm and own:
                loop = own
                if hm.group(1) == "1":
                    depth1.add(own)
                children[own] = re.findall(r"Child Loop (BB\d+_\d+) Depth", note)
            else:
                im = re.search(r"in Loop: Header=(BB\d+_\d+) Depth=\d+", note)
                loop = im.group(1) if im else None
            cur = {"loop": loop, "lines": []}
            blocks.append(cur)
            continue
        if cur is not None:
            cur["lines"].append(l)

    def nest(h):
        out = {h}
        for c in children.get(h, []):
            out |= nest(c)
        return out

    if not depth1:
        return {"path": (0, 0, 0), "off": (0, 0, 0)}
    sizes = {h: sum(b["loop"] in nest(h) for b in blocks) for h in depth1}
    main = nest(max(sizes, key=sizes.get))
    res = {"path": [0, 0, 0], "off": [0, 0, 0]}
    for b in blocks:
        if b["loop"] not in main:
            continue
        body = b["lines"]
        off = any(("global_atomic" in x or "s_memrealtime" in x) for x in body)
        k = "off" if off else "path"
        res[k][0] += sum("v_readlane_b32" in x for x in body)
        res[k][1] += sum("v_writelane_b32" in x for x in body)
        res[k][2] += sum(re.search(r"\bscratch_(load|store)", x) is not None for x in body)
    return {k: tuple(v) for k, v in res.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None)
    ap.add_argument("--match", nargs="*", default=list(DEFAULT_MATCH))
    a = ap.parse_args()
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            results = list(ex.map(lambda s: compile_one(s, tmp), SOURCES))
        rows = []
        for src, remarks, asm in results:
            rem = parse_remarks(remarks)
            text = open(asm).read() if asm else ""
            dm = demangle(list(rem))
            for fn, r in rem.items():
                name = dm.get(fn, fn)
                if not any(m in name for m in a.match):
                    continue
                mv = loop_moves(text, fn) if text else None
                rows.append((src, name, r, mv))
    out = ["# register use of the path's kernels (compiler resource remarks, gfx950)", "",
           "command:", "", "    python -m layer_lstm_amd.kernel_resources" +
           (f" --out {a.out}" if a.out else ""), "",
           "per kernel: VGPRs AGPRs SGPRs | SGPRs spilled, VGPRs spilled, scratch bytes/lane | in the step loop, "
           "per-step path: readlane/writelane/scratch instructions; failure and stamp paths: the same", ""]
    for src, name, r, mv in sorted(rows, key=lambda x: (x[0], x[1])):
        short = re.sub(r"\(lstm::.*$", "", name)
        short = short.replace("void lstm::", "").replace("unsigned short", "u16")
        short = re.sub(r"lstm::", "", short)
        if len(short) > 110:
            short = short[:107] + "..."
        p = mv["path"] if mv else ("-", "-", "-")
        o = mv["off"] if mv else ("-", "-", "-")
        out.append(f"{short}")
        out.append(f"    regs {r.get('vgpr', 0):3d} v {r.get('agpr', 0):3d} a {r.get('sgpr', 0):3d} s | spills "
                   f"s {r.get('sgpr_spill', 0):3d} v {r.get('vgpr_spill', 0):3d} scratch {r.get('scratch', 0):3d} B | "
                   f"step loop: path {p[0]}/{p[1]}/{p[2]}  failure+stamp paths {o[0]}/{o[1]}/{o[2]}")
    text = "\n".join(out) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
