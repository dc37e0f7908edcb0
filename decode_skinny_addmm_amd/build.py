"""Ahead-of-time build of libskinny.so for gfx950 with hipcc (no JIT at run time).

    python -m decode_skinny_addmm_amd.build      # or __graft_entry__.build()

Every .hip file in csrc/ is compiled to an object in parallel, then linked into
decode_skinny_addmm_amd/libskinny.so. Packed-fp32 instructions are disabled for all
device code (-packed-fp32-ops). kernel_code.json beside the library maps each kernel's
mangled name to a hash of its gfx950 machine code (the key of measured byte counts).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libskinny.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm install expected under /opt/rocm)")


def common_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stderr or "").splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


CODE_MAP = os.path.join(PKG, "kernel_code.json")


def _llvm(tool: str) -> str:
    for d in ("/opt/rocm/lib/llvm/bin", "/opt/rocm/llvm/bin"):
        if os.path.exists(os.path.join(d, tool)):
            return os.path.join(d, tool)
    found = shutil.which(tool)
    if not found:
        raise RuntimeError("%s not found (ROCm LLVM tools expected under /opt/rocm)" % tool)
    return found


def _code_objects(lib: str) -> list[bytes]:
    """The gfx950 code objects in the library's .hip_fatbin section: one offload bundle per
    translation unit (magic, entry count, then offset/size/triple per entry)."""
    import struct
    import tempfile
    with tempfile.TemporaryDirectory() as td:
        sec = os.path.join(td, "fatbin")
        subprocess.run([_llvm("llvm-objcopy"), "--dump-section", ".hip_fatbin=" + sec, lib, os.devnull], check=True)
        data = open(sec, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out, pos = [], data.find(magic)
    while pos >= 0:
        n = struct.unpack_from("<Q", data, pos + len(magic))[0]
        q = pos + len(magic) + 8
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", data, q)
            triple = data[q + 24:q + 24 + tlen].decode()
            q += 24 + tlen
            if triple.endswith(ARCH) or ("--" + ARCH) in triple:
                out.append(data[pos + off:pos + off + size])
        pos = data.find(magic, pos + 1)
    return out


def kernel_code_hashes(lib: str = LIB) -> dict:
    """Mangled kernel name -> SHA-256 of its machine code, over every gfx950 code object in the
    library. A measurement keyed by this hash (profiles/traffic.json) goes stale exactly when
    that kernel's code changes."""
    import hashlib
    import tempfile
    res = {}
    for co in _code_objects(lib):
        with tempfile.NamedTemporaryFile(suffix=".co") as f:
            f.write(co)
            f.flush()
            secs = subprocess.run([_llvm("llvm-readelf"), "-S", "-W", f.name], capture_output=True, text=True,
                                  check=True).stdout
            syms = subprocess.run([_llvm("llvm-readelf"), "-s", "-W", f.name], capture_output=True, text=True,
                                  check=True).stdout
        text = None
        for line in secs.splitlines():
            parts = line.replace("[ ", "[").split()
            if len(parts) > 6 and parts[1] == ".text":
                text = (int(parts[3], 16), int(parts[4], 16))   # address, file offset
        if text is None:
            continue
        for line in syms.splitlines():
            parts = line.split()
            if len(parts) >= 8 and parts[3] == "FUNC" and parts[7].startswith("_Z"):
                addr, size = int(parts[1], 16), int(parts[2])
                start = text[1] + addr - text[0]
                res[parts[7]] = hashlib.sha256(co[start:start + size]).hexdigest()
    # the demangled names too (the form profilers report), when a demangler is installed
    demangler = shutil.which("llvm-cxxfilt") or shutil.which("c++filt")
    if demangler:
        names = sorted(res)
        dem = subprocess.run([demangler], input="\n".join(names), capture_output=True, text=True,
                             check=True).stdout.splitlines()
        for m, d in zip(names, dem):
            if d != m:
                res[d] = res[m]
    return res


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    import json
    with open(CODE_MAP + ".tmp", "w") as f:
        json.dump(kernel_code_hashes(LIB), f, indent=0, sort_keys=True)
    os.replace(CODE_MAP + ".tmp", CODE_MAP)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build()
