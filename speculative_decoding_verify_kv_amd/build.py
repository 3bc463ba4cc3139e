"""Build libverify_attn.so in-tree with hipcc for gfx950.

Each HIP source is compiled to an object in parallel, then linked into one
shared library next to this file.  Packed fp32 VALU forms are disabled for
the device code.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libverify_attn.so")
SOURCES = ["api.hip", "verify_partial.hip", "verify_merge.hip", "ragged_schedule.hip", "append_kv.hip",
           "promote_kv.hip"]
# The partial kernel keeps its O accumulators in VGPRs and lets the Q operand
# fragments sit in AGPRs (MFMA reads A/B from AGPRs); the default heuristic
# instead shuttles the accumulators through AGPR spill slots every iteration.
# Its instructions are scheduled for instruction-level parallelism rather
# than occupancy (the kernel runs one workgroup per CU whatever the
# schedule): 0.2-0.4 us less per launch, the same registers and results.
# Its first seven kernel arguments (what a workgroup needs to issue its Q
# copies) are preloaded into SGPRs at wave launch.
PER_SOURCE_FLAGS = {"verify_partial.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1",
                                           "-mllvm", "-amdgpu-sched-strategy=max-ilp",
                                           "-mllvm", "-amdgpu-kernarg-preload-count=7"],
                    "verify_merge.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=5"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    ]


def _compile(src: str, obj: str, extra=()):
    cmd = [hipcc(), *_flags(), *PER_SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    return warn


def build(verbose: bool = False, extra=()) -> str:
    """Compile every HIP source for gfx950 and link libverify_attn.so (always rebuilds)."""
    with tempfile.TemporaryDirectory(prefix="va_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
        with cf.ThreadPoolExecutor(jobs) as ex:
            futs = [ex.submit(_compile, s, o, extra) for s, o in zip(SOURCES, objs)]
            for f in futs:
                w = f.result()
                if verbose and w:
                    print(w, file=sys.stderr)
        out_tmp = LIB + ".tmp%d" % os.getpid()
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr[-4000:])
        os.replace(out_tmp, LIB)
    return LIB


def resource_report() -> str:
    """Per-kernel register, scratch, LDS and occupancy figures the compiler
    reports for the gfx950 code of every source (a markdown table)."""
    import re

    rows = []
    with tempfile.TemporaryDirectory(prefix="va_res_") as tmp:
        for src in SOURCES:
            cmd = [hipcc(), *_flags(), *PER_SOURCE_FLAGS.get(src, []), "--cuda-device-only", "-c",
                   os.path.join(CSRC, src), "-o", os.path.join(tmp, src + ".o"),
                   "-Rpass-analysis=kernel-resource-usage"]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
            cur = None
            for line in r.stderr.splitlines():
                m = re.search(r"remark: Function Name: (\S+)", line)
                if m:
                    cur = {"src": src, "name": m.group(1)}
                    rows.append(cur)
                    continue
                m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
                if m and cur is not None:
                    cur[m.group(1).strip()] = m.group(2)
    names = subprocess.run(["c++filt"], input="\n".join(r["name"] for r in rows), capture_output=True,
                           text=True).stdout.splitlines() if shutil.which("c++filt") else [r["name"] for r in rows]
    out = ["| kernel | source | VGPR | AGPR | SGPR | VGPR spill | SGPR spill | scratch B/lane | LDS B/block |"
           " waves/SIMD |", "|---|---|---|---|---|---|---|---|---|---|"]
    for r, n in zip(rows, names):
        n = n.replace("va::(anonymous namespace)::", "").replace("(va::PartialParams)", "").replace(
            "(va::MergeParams)", "").replace("(va::ScheduleParams)", "").replace("(va::AppendParams)", "").replace("(va::PromoteParams)", "")
        out.append(f"| `{n}` | {r['src']} | {r.get('VGPRs')} | {r.get('AGPRs')} | {r.get('TotalSGPRs')} | "
                   f"{r.get('VGPRs Spill')} | {r.get('SGPRs Spill')} | {r.get('ScratchSize')} | {r.get('LDS Size')} | "
                   f"{r.get('Occupancy')} |")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resources":
        print(resource_report())
    else:
        print(build(verbose=True))
