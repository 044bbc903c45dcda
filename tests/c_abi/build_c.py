"""Compile the standalone C consumer of the C ABI (tests/c_abi/fvattn_path.c)
with gcc against include/fvattn.h and the in-tree libfvattn.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "fvattn_path.c")
BIN = os.path.join(HERE, "fvattn_path")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    pkg = os.path.join(ROOT, "block_sparse_attention_11_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", SRC, "-o", BIN,
           f"-L{pkg}", "-lfvattn", f"-L{ROCM}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../block_sparse_attention_11_amd", f"-Wl,-rpath,{ROCM}/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed:\n{res.stdout}\n{res.stderr}")
    if verbose:
        print(f"built {BIN}")
    return BIN


if __name__ == "__main__":
    build(verbose=True)
