"""Build libpa.so (HIP, gfx950) in-tree.

    python -m paged_kv_cache_157_amd.build

Every source is compiled with hipcc for gfx950 only; packed fp32 VALU forms
are disabled.  Objects are compiled in parallel and linked into
paged_kv_cache_157_amd/libpa.so next to this file.

Guards (the build fails, before linking, when one trips):
  * any inline-assembly warning (-Werror=inline-asm): a reserved register on
    a clobber list, for instance, is undefined behaviour;
  * any kernel with scratch memory, a dynamic stack or spilled VGPRs (read
    from the compiler's kernel-resource-usage remarks).  The decode and
    prefill kernels count their own global->LDS loads with hand-written
    `s_waitcnt vmcnt(N)` waits, which are correct only while no other vector
    memory instruction (a scratch spill or reload is one) interleaves with
    those loads.  SGPR spills are allowed while the scratch size is zero:
    they then live in VGPR lanes (v_writelane / v_readlane) and issue no
    memory instruction.
The per-kernel register and scratch figures are written to
_build/resource_usage.txt.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpa.so")
SOURCES = ["decode_hg4.hip", "decode.hip", "prefill.hip", "reshape.hip", "copy_blocks.hip",
           "pa_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Wall", "-Wno-unused-function", "-Werror=inline-asm",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


_REMARK = re.compile(r"remark:\s+(Function Name|TotalSGPRs|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|"
                     r"Dynamic Stack|Occupancy \[waves/SIMD\]|SGPRs Spill|VGPRs Spill|"
                     r"LDS Size \[bytes/block\]): (\S+)")
_KEYS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr", "ScratchSize [bytes/lane]": "scratch",
         "Dynamic Stack": "dynstack", "Occupancy [waves/SIMD]": "occupancy",
         "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill", "LDS Size [bytes/block]": "lds"}


def resource_usage(stderr: str):
    """Per-kernel records parsed from -Rpass-analysis=kernel-resource-usage remarks."""
    recs, cur = [], None
    for m in _REMARK.finditer(stderr):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = {"name": val}
            recs.append(cur)
        elif cur is not None:
            cur[_KEYS[key]] = val
    return recs


def _compile(src: str, obj_dir: str, defines=()):
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = ([hipcc()] + common_flags() + [f"-D{d}" for d in defines] +
           ["-Rpass-analysis=kernel-resource-usage", "-c"] + lang +
           [os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    lines = [l for l in (r.stderr or "").splitlines() if noise not in l]
    usage = resource_usage("\n".join(lines))
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l and not
                    re.match(r"^\s*(\d+ \|.*|\|\s*\^?)\s*$", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if "warning:" in err or "error:" in err:
        sys.stderr.write(err + "\n")
    return obj, [dict(u, source=src) for u in usage]


def _demangle(names):
    try:
        r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
        out = r.stdout.splitlines()
        if r.returncode == 0 and len(out) == len(names):
            return out
    except OSError:
        pass
    return list(names)


def check_resources(usage, obj_dir: str, verbose: bool) -> None:
    """Write the per-kernel table and refuse kernels with scratch, a dynamic
    stack or spills."""
    kernels = [u for u in usage if "vgpr" in u]
    names = _demangle([u["name"] for u in kernels])
    bad = []
    rows = ["source\tvgpr\tagpr\tsgpr\tscratch\tvgpr_spill\tsgpr_spill\tlds\toccupancy\tkernel"]
    for u, nm in zip(kernels, names):
        rows.append("\t".join([u["source"], u["vgpr"], u.get("agpr", "0"), u.get("sgpr", "?"),
                               u.get("scratch", "?"), u.get("vgpr_spill", "?"),
                               u.get("sgpr_spill", "?"), u.get("lds", "?"),
                               u.get("occupancy", "?"), nm]))
        if u.get("scratch") != "0" or u.get("dynstack") != "False" or u.get("vgpr_spill") != "0":
            bad.append(f"{nm} ({u['source']}): scratch {u.get('scratch')} B/lane, dynamic stack "
                       f"{u.get('dynstack')}, VGPR spills {u.get('vgpr_spill')}")
    with open(os.path.join(obj_dir, "resource_usage.txt"), "w") as f:
        f.write("\n".join(rows) + "\n")
    if verbose:
        by_src = {}
        for u in kernels:
            by_src.setdefault(u["source"], []).append(u)
        for src, us in sorted(by_src.items()):
            print(f"  {src}: {len(us)} kernels, VGPRs <= {max(int(u['vgpr']) for u in us)}, "
                  f"AGPRs <= {max(int(u.get('agpr', 0)) for u in us)}, scratch "
                  f"{max(int(u.get('scratch', 0)) for u in us)} B/lane, VGPR spills "
                  f"{sum(int(u.get('vgpr_spill', 0)) for u in us)}, SGPRs spilled to VGPR lanes "
                  f"<= {max(int(u.get('sgpr_spill', 0)) for u in us)}")
    if not kernels:
        raise RuntimeError("no kernel-resource-usage remarks found: cannot check for scratch")
    if bad:
        raise RuntimeError("kernels with scratch memory or VGPR spills (their hand-counted "
                           "vmcnt waits would be wrong):\n  " + "\n  ".join(bad))


def build(verbose: bool = True, defines=(), out: str = LIB) -> str:
    """Compile every source and link `out` (default: the in-tree libpa.so).
    `defines` are extra -D switches (tuning constants such as DECODE_STAGES)."""
    obj_dir = os.path.join(HERE, "_build" if not defines else "_build_" + "_".join(defines))
    os.makedirs(obj_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(6, len(SOURCES))) as ex:
        res = list(ex.map(lambda s: _compile(s, obj_dir, defines), SOURCES))
    objs = [o for o, _ in res]
    check_resources([u for _, us in res for u in us], obj_dir, verbose)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link of libpa.so failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
