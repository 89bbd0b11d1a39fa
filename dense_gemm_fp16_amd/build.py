"""Build libgemm_tn.so (the HIP kernels and the C ABI) for gfx950 in-tree.

    python dense_gemm_fp16_amd/build.py [--defines GTN_T256_MFMA=32 ...]

(run as a script: importing the package itself needs the built library).

Each translation unit under csrc/ is compiled by hipcc in parallel, then
linked into dense_gemm_fp16_amd/libgemm_tn.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libgemm_tn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # code object v5: loadable by the HIP runtime that ships inside torch
    "-mcode-object-version=5",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


# Per-file flags.  The attention kernel (the softmax, the rescale by a new
# row maximum) and the fp16-accumulating GEMM (the fp16 rounding after every
# step) apply vector ALU work to MFMA results; with the MFMA operands and
# results in ordinary VGPRs instead of accumulation registers, none of that
# costs a copy between the two register files.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
FILE_FLAGS = {
    "attention_fwd.hip": _VGPR_FORM,
    "gemm_f16acc.hip": _VGPR_FORM,
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip"))


def _compile(src, obj, extra):
    cmd = ([HIPCC] + FLAGS + FILE_FLAGS.get(os.path.basename(src), [])
           + extra + ["-c", src, "-o", obj])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True)
    # hipcc's host pass does not know the device-only feature; drop that note
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return out


def build(defines=(), out_path=LIB_PATH, jobs=None, save_temps=False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = ["-D" + d for d in defines]
    if save_temps:
        extra.append("--save-temps")
    tag = "_".join(d.replace("=", "") for d in defines) or "default"
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, os.cpu_count() or 1)) as ex:
        futs = []
        for src in sources():
            obj = os.path.join(BUILD_DIR, f"{os.path.basename(src)}.{tag}.o")
            objs.append(obj)
            futs.append(ex.submit(_compile, src, obj, extra))
        for f in futs:
            msg = f.result()
            if msg.strip():
                print(msg, file=sys.stderr)
    tmp = out_path + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH,
                           "-mcode-object-version=5", "-shared", "-fPIC",
                           "-o", tmp] + objs)
    os.replace(tmp, out_path)
    return out_path


FAST_NAME = "_gemm_tn_fast"
FAST_PATH = os.path.join(PKG, FAST_NAME + ".so")


def build_fast_binding() -> str:
    """The binding's fast path (csrc/binding_fast.cpp, host C++ against
    torch's headers, no HIP): built with torch.utils.cpp_extension into
    _build/, then placed next to the library.  The package imports it when
    present and otherwise marshals through ctypes."""
    import shutil
    from torch.utils import cpp_extension
    bdir = os.path.join(BUILD_DIR, "fast_binding")
    os.makedirs(bdir, exist_ok=True)
    cpp_extension.load(name=FAST_NAME,
                       sources=[os.path.join(CSRC, "binding_fast.cpp")],
                       extra_cflags=["-O2", "-I" + os.path.join(ROOT,
                                                                "include")],
                       build_directory=bdir, with_cuda=False,
                       is_python_module=True, verbose=False)
    built = os.path.join(bdir, FAST_NAME + ".so")
    tmp = FAST_PATH + ".tmp%d" % os.getpid()
    shutil.copyfile(built, tmp)
    os.replace(tmp, FAST_PATH)
    return FAST_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--defines", nargs="*", default=[])
    ap.add_argument("--out", default=LIB_PATH)
    ap.add_argument("--save-temps", action="store_true")
    a = ap.parse_args()
    print(build(a.defines, a.out, save_temps=a.save_temps))
