"""Build libwts.so (gfx950) in-tree with hipcc.

    python -m serial_draft_head_persistent_amd.build [-v] [--resources]

Both translation units are compiled as HIP for gfx950 only.  Flags that the
numerics depend on: -ffp-contract=off (no fused a*b+c, so every binary32
operation rounds once, as the host reference assumes); packed fp32 vector
instructions disabled.

The kernels are compiled with the compiler's resource-usage remarks; their
registers, scratch and spill counts per kernel are written next to the
library (libwts.resources.json).  A spill in a walk kernel means W tiles or
working values that were meant to stay in registers go through scratch
memory: the register/LDS placement of the shard (Fig. 12) is then wrong.
--resources prints them as a table.
"""
import json
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwts.so")
RESOURCES = os.path.join(PKG, "libwts.resources.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["wts_kernels.hip", "wts_runtime.hip", "wts_roofline.hip"]
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


_FIELDS = {"VGPRs": "vgpr", "AGPRs": "agpr", "SGPRs": "sgpr", "ScratchSize [bytes/lane]": "scratch",
           "VGPRs Spill": "vgpr_spill", "SGPRs Spill": "sgpr_spill", "Occupancy [waves/SIMD]": "occupancy",
           "LDS Size [bytes/block]": "static_lds"}


def kernel_label(mangled):
    """walk_kernel<wtype, batch bucket, head, T, lse> style label of a mangled kernel name."""
    m = re.match(r"_ZN3wts\d+(\w+?)I(.*)EEvNS_8WalkArgsE", mangled)
    if not m:
        m2 = re.match(r"_ZN3wts\d+(\w+?)E", mangled)
        return m2.group(1) if m2 else mangled
    args = re.findall(r"L([ib])(\d+)E", m.group(2))
    return f"{m.group(1)}<{', '.join(v if t == 'i' else ('true' if v == '1' else 'false') for t, v in args)}>"


def parse_resources(text):
    """Per-kernel resource usage from -Rpass-analysis=kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = kernel_label(m.group(1))
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?): (\w+)", line)
        if cur and m and m.group(1) in _FIELDS:
            v = m.group(2)
            out[cur][_FIELDS[m.group(1)]] = int(v) if v.isdigit() else v
    return out


def build(verbose=False, jobs=3):
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        extra = ["-Rpass-analysis=kernel-resource-usage"] if src == "wts_kernels.hip" else []
        cmd = [HIPCC] + FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), src))
        objs.append(obj)
    resources = {}
    for pr, src in procs:
        out = pr.communicate()[0].decode(errors="replace")
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{out}")
        resources.update(parse_resources(out))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    with open(RESOURCES, "w") as fh:
        json.dump(resources, fh, indent=1, sort_keys=True)
    return LIB


def resource_table(resources):
    rows = ["| kernel | VGPR | AGPR | scratch B/lane | VGPR spills | waves/SIMD |", "|---|---|---|---|---|---|"]
    def order(k):
        name, _, rest = k.partition("<")
        return name, [int(x) if x.strip().isdigit() else x.strip() for x in rest.rstrip(">").split(",")]
    for k in sorted(resources, key=order):
        r = resources[k]
        if "walk_kernel" in k or "step_kernel" in k:
            rows.append(f"| `{k}` | {r.get('vgpr')} | {r.get('agpr')} | {r.get('scratch')} | "
                        f"{r.get('vgpr_spill')} | {r.get('occupancy')} |")
    return "\n".join(rows)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--resources" in sys.argv:
        with open(RESOURCES) as fh:
            print(resource_table(json.load(fh)))
