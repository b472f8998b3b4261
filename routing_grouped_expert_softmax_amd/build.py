"""Build libmoe_amd.so from the HIP sources for gfx950 (hipcc, one object per source,
compiled in parallel, then linked). Run as `python routing_grouped_expert_softmax_amd/build.py`
(by path: importing the package itself loads the built library).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_amd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.hip", "route.hip", "permute.hip", "combine.hip", "grouped_gemm.hip",
           "grouped_gemm_bwd.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed-fp32 instructions: plain fp32 arithmetic only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def resource_usage() -> str:
    """Recompile every source with the compiler's kernel-resource-usage remarks (nothing is
    linked or replaced) and return one line per kernel: VGPRs, AGPRs, SGPRs, spilled VGPRs
    and SGPRs, scratch bytes per lane, LDS bytes per block (static; the GEMMs add dynamic
    LDS at launch) and waves per SIMD the registers allow."""
    import re
    import tempfile
    rows = []
    keys = {"VGPRs": "vgpr", "AGPRs": "agpr", "TotalSGPRs": "sgpr", "VGPRs Spill": "vspill",
            "SGPRs Spill": "sspill", "ScratchSize [bytes/lane]": "scratch",
            "LDS Size [bytes/block]": "lds", "Occupancy [waves/SIMD]": "occ"}
    pat = re.compile(r"remark:\s+(Function Name|[A-Za-z ]+(?:\[[^\]]*\])?):\s*(\S+)")
    with tempfile.TemporaryDirectory() as tmp:
        for src in SOURCES:
            cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c",
                                     os.path.join(CSRC, src), "-o", os.path.join(tmp, "k.o")]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
            cur = None
            for line in r.stderr.splitlines():
                m = pat.search(line)
                if not m:
                    continue
                k, v = m.group(1).strip(), m.group(2)
                if k == "Function Name":
                    cur = {"src": src, "name": v}
                    rows.append(cur)
                elif cur is not None and k in keys:
                    cur[keys[k]] = v
    try:                                    # demangled names where c++filt is present
        names = subprocess.run(["c++filt"], input="\n".join(r["name"] for r in rows),
                               text=True, capture_output=True).stdout.splitlines()
        if len(names) == len(rows):
            for r, n in zip(rows, names):
                r["name"] = n
    except OSError:
        pass
    for r in rows:                          # short names: no namespace, return type, arguments
        n = r["name"].replace("moe::(anonymous namespace)::", "").replace("moe::", "")
        n = n[5:] if n.startswith("void ") else n
        r["name"] = n.split("(")[0]
    cols = ["vgpr", "agpr", "sgpr", "vspill", "sspill", "scratch", "lds", "occ"]
    out = ["source | " + " | ".join(cols) + " | kernel"]
    for r in rows:
        out.append(f"{r['src']} | " + " | ".join(str(r.get(c, "?")) for c in cols) +
                   f" | {r['name']}")
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage())
    else:
        build(verbose=True)
    sys.exit(0)
