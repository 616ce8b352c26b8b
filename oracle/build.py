"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain C compiled by gcc with no fast-math and no floating-point contraction, so
the fp32 routing key of the sigmoid router is exactly the written sequence of
fp32 operations.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, sanitize: bool = False, out: str = None) -> str:
    """sanitize: AddressSanitizer + UndefinedBehaviorSanitizer build (load it
    with gcc's libasan preloaded), written to `out`."""
    lib = out or LIB
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wno-unknown-pragmas",
    ]
    if sanitize:
        cmd += ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    cmd += [SRC, "-o", lib + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
