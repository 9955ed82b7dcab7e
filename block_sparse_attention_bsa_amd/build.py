"""Build the HIP library libbsa.so for gfx950 in-tree (block_sparse_attention_bsa_amd/_lib/).

Every source under csrc/ is compiled by hipcc in one invocation. Packed-fp32 instruction
selection is disabled for device code (the compiler's own v_pk_*_f32 forms are avoided).
"""
import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBDIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIBDIR, "libbsa.so")
ARCH = os.environ.get("BSA_OFFLOAD_ARCH", "gfx950")


INCLUDE = os.path.join(HERE, "..", "include")
STAMP = LIB + ".srchash"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def source_hash():
    """sha256 over every file the library is built from (csrc/ and include/), with names."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    files += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    for path in sorted(f for f in files if f.endswith((".hip", ".cpp", ".h"))):
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", os.path.join(HERE, "..", "include"),
           "-o", tmp] + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed building libbsa.so")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    with open(STAMP, "w") as f:  # which sources this library was built from (checked at load)
        f.write(source_hash() + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
