"""Build libkvdec.so in-tree with hipcc for gfx950.

    python -m long_context_decode_kv_amd.build

Every translation unit is compiled for gfx950 with the packed-fp32 VALU
operations switched off (hipcc's host pass warns that it does not know the
feature; that is harmless).  The objects go to ``_build/`` at the repository
root, the library to ``long_context_decode_kv_amd/libkvdec.so`` and the
streaming-read probe used by the benchmark to ``libkvprobe.so`` beside it.
"""

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvdec.so")

SOURCES = ["kernels.hip", "split_f16.hip", "split_q8.hip", "split_q4.hip", "split_f16_q8.hip", "split_f16_q4.hip",
           "split_q8_q4.hip", "plan_device.hip", "static_scratch.hip", "api.cpp", "plan.cpp"]
# the streaming-read probe (bandwidth ceiling for the benchmark) is a library of its own
PROBE_SOURCES = ["probe.hip"]
PROBE_LIB = os.path.join(PKG, "libkvprobe.so")
# test build: the same objects, api.cpp compiled with KVDEC_FAULT_INJECTION
# (host-side failure injection of the tail streamer) plus its switches
FI_LIB = os.path.join(PKG, "libkvdec_fi.so")
FI_SOURCES = ["fault_injection.hip"]
# test build: the planner and the C-ABI validation (plan.cpp, api.cpp) with
# AddressSanitizer and UndefinedBehaviorSanitizer on the host side, linked
# with the ordinary device objects; loaded with the ASan runtime preloaded
SAN_LIB = os.path.join(PKG, "libkvdec_san.so")
SAN_HOST = ["plan.cpp", "api.cpp"]
# diagnostic build: every source compiled with KVDEC_PHASE_TRACE -- the
# one-shot kernel and its merge write clock stamps of their phases to a
# buffer given through kvdec_trace_configure (long_context_decode_kv_amd.phase_trace)
TRACE_LIB = os.path.join(PKG, "libkvdec_trace.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the O tile is rescaled by
    # VALU code, which cannot address accumulation registers directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]

# Flags of single sources.  The int8 K / int8 V matrix-core kernels keep their
# loads in clauses under the memory-clause scheduling strategy: the 4-slot
# GQA-6 int8 step measured 2-3% shorter in five A/B pairs (104.4 -> 101.3,
# 106.9 -> 104.5 us); the same strategy on the other storage pairs measured
# slower (int8 K / 4-bit V +4%) or no different, so they keep the default.
SOURCE_FLAGS = {
    "split_q8.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
}


def source_hash():
    """16 hex digits of sha256 over every source the libraries are built
    from (csrc/, include/) and the compiler flags: the value the library
    embeds and the binding checks at import."""
    import hashlib
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))]
    inc = os.path.join(ROOT, "include")
    files += [os.path.join(inc, f) for f in sorted(os.listdir(inc))]
    for f in files:
        if os.path.isfile(f) and f.endswith((".h", ".hip", ".cpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    h.update(" ".join(FLAGS[:-4]).encode())  # the flags without the two -I paths
    h.update(repr(sorted(SOURCE_FLAGS.items())).encode())
    return h.hexdigest()[:16]


def hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


# Kernel resource remarks: a kernel that needs per-lane scratch (a spilled
# or dynamically indexed register array) fails the build -- on these kernels
# it has meant a many-fold slowdown, never a valid trade.
RESOURCE_REMARKS = ["-Rpass-analysis=kernel-resource-usage"]


def _scratch_kernels(log):
    """(kernel, bytes per lane) for every kernel the remarks show using scratch."""
    found, name = [], None
    for line in log.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    return found


def _compile(src, extra, suffix=""):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    remarks = RESOURCE_REMARKS if src.endswith(".hip") else []
    cmd = [hipcc()] + lang + FLAGS + SOURCE_FLAGS.get(src, []) + remarks + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    spills = _scratch_kernels(r.stderr)
    if spills:
        raise RuntimeError(f"{src}: kernels using scratch memory: {spills}")
    log = "\n".join(line for line in r.stderr.splitlines() if "remark:" not in line)
    return obj, log


HASH_FILE = LIB + ".srchash"


def build(verbose=False, extra=()):
    os.makedirs(BUILD, exist_ok=True)
    digest = source_hash()
    hash_def = ['-DKVDEC_SOURCE_HASH="%s"' % digest]
    jobs = [(s, list(extra) + hash_def, "") for s in SOURCES + PROBE_SOURCES + FI_SOURCES]
    jobs.append(("api.cpp", list(extra) + hash_def + ["-DKVDEC_FAULT_INJECTION"], "_fi"))
    jobs += [(h, list(extra) + hash_def + SAN_FLAGS, "_san") for h in SAN_HOST]
    jobs += [(s, list(extra) + hash_def + ["-DKVDEC_PHASE_TRACE"], "_tr") for s in SOURCES]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 8)) as ex:
        outs = list(ex.map(lambda j: _compile(*j), jobs))
    results = {j[0] + j[2]: o for j, o in zip(jobs, outs)}
    if verbose:
        for _, log in results.values():
            if log.strip():
                print(log, file=sys.stderr)
    fi_names = [n for n in SOURCES if n != "api.cpp"] + ["api.cpp_fi"] + FI_SOURCES
    san_names = [n for n in SOURCES if n not in SAN_HOST] + [h + "_san" for h in SAN_HOST]
    san_link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    tr_names = [n + "_tr" for n in SOURCES]
    for lib, names, link in ((LIB, SOURCES, []), (PROBE_LIB, PROBE_SOURCES, []), (FI_LIB, fi_names, []),
                             (SAN_LIB, san_names, san_link), (TRACE_LIB, tr_names, [])):
        tmp = lib + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + link + ["-o", tmp] + [results[n][0] for n in names]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, lib)
    with open(HASH_FILE, "w") as fh:
        fh.write(digest + "\n")
    return LIB


def asan_runtime():
    """Path of the compiler's shared AddressSanitizer runtime (to preload
    when loading the sanitizer build into an uninstrumented interpreter)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def built_hash():
    """The source hash recorded beside the built library, or None."""
    try:
        with open(HASH_FILE) as fh:
            return fh.read().strip()
    except OSError:
        return None


def ensure_built():
    """Build when the libraries are missing or were built from other
    sources than the current ones (the recorded source hash differs)."""
    if not all(os.path.exists(x) for x in (LIB, PROBE_LIB, FI_LIB, SAN_LIB, TRACE_LIB)) or \
            built_hash() != source_hash():
        build()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
