"""Build libdstopk.so in place with hipcc for gfx950 (one shared library: kernels + C ABI).

The device code is instantiated by several translation units (the select kernels once per
element type and counter mode, then the merge kernels and probes), which compile in
parallel and link into the one library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
OUT = os.path.join(HERE, "libdstopk.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # never let the compiler form packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # LDS atomics here are issued by one lane on purpose; the atomic optimizer's wave
    # reduction around them only adds instructions
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]

# (object name, source, extra flags)
# (the select and list-merge kernels' leading scalar arguments are preloaded into SGPRs)
UNITS = [(f"select_{dt}{'_stats' if st else ''}{'_ext' if ex else ''}", "ds_select.hip",
          [f"-DDS_PART_DT={d}", f"-DDS_PART_STATS={st}", f"-DDS_PART_EXT={ex}",
           "-mllvm", "-amdgpu-kernarg-preload-count=15"])
         for d, dt in ((0, "bf16"), (1, "fp32")) for st in (0, 1) for ex in (0, 1)] + [
    ("merge", "ds_merge.hip", ["-mllvm", "-amdgpu-kernarg-preload-count=14"]),
    ("noalloc", "ds_noalloc.hip", []),
    ("api", "ds_api.cpp", [])]

NOISE = "packed-fp32-ops"


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msgs = [l for l in res.stdout.splitlines() if NOISE not in l and l.strip()]
    return res.returncode, msgs


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (the device code is built as
# usual): a separate library for checking the host code, loaded through DS_LIBRARY with the
# clang ASan runtime preloaded.
HOST_SANITIZERS = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build(verbose: bool = False, jobs: int = 0, out: str = OUT, extra_flags=()) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    flags = FLAGS + list(extra_flags)
    cmds = []
    objs = []
    for name, src, extra in UNITS:
        obj = os.path.join(OBJDIR, f"{name}.{tag}.o")
        objs.append(obj)
        cmds.append([HIPCC] + flags + extra + ["-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, msgs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            failed = True
            sys.stderr.write("\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
        raise RuntimeError("hipcc failed")
    tmp = out + ".tmp" + tag
    rc, msgs = _run([HIPCC] + flags + ["-shared", "-o", tmp] + objs)
    for o in objs:
        os.remove(o)
    if rc != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc link failed ({rc})")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libdstopk.so for gfx950")
    ap.add_argument("--host-sanitizers", metavar="LIB",
                    help="build a copy with host-side ASan/UBSan at LIB instead of the library in place")
    args = ap.parse_args()
    if args.host_sanitizers:
        print(build(verbose=True, out=os.path.abspath(args.host_sanitizers), extra_flags=HOST_SANITIZERS))
    else:
        print(build(verbose=True))
