"""Compile the plain C consumer of libhybrid_attn.so (gcc, host code only).

It links the in-tree library and the C oracle (test code) by rpath, so it runs
from the tree without an install step.  Build both libraries first.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_consumer.c")
EXE = os.path.join(HERE, "abi_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_consumer(out: str = EXE) -> str:
    lib_dir = os.path.join(ROOT, "block_hybrid_linear_amd")
    oracle_dir = os.path.join(ROOT, "oracle")
    rel = lambda p: os.path.relpath(p, os.path.dirname(os.path.abspath(out)))  # noqa: E731
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), SRC, "-o", out,
           "-L", lib_dir, "-lhybrid_attn", "-L", oracle_dir, "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,$ORIGIN/{rel(lib_dir)}", f"-Wl,-rpath,$ORIGIN/{rel(oracle_dir)}",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed for {SRC}:\n{r.stdout}\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build_consumer())
