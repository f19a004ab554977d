"""Compile the C oracle (``latentmoe_oracle.c``) into ``liblatentmoe_oracle.so``.

Test infrastructure only.  Plain gcc, fp64, no fast-math, no FMA contraction.
``build(sanitize=True)`` builds ``liblatentmoe_oracle_san.so`` instead, with
AddressSanitizer and UndefinedBehaviorSanitizer (every UB report aborts); a
process loads it with the ASan runtime preloaded (``sanitizer_env()``) and
``LATENTMOE_ORACLE_LIB`` naming it.
"""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "latentmoe_oracle.c")
LIB = os.path.join(HERE, "liblatentmoe_oracle.so")
SAN_LIB = os.path.join(HERE, "liblatentmoe_oracle_san.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2" if not sanitize else "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"] + (SAN_FLAGS if sanitize else []) + \
        ["-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def sanitizer_env(base=None) -> dict:
    """Environment of a process that loads the sanitized oracle: the ASan
    runtime preloaded (the interpreter itself is not instrumented), leak
    checks off (the interpreter's own allocations would be reported)."""
    env = dict(os.environ if base is None else base)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["LATENTMOE_ORACLE_LIB"] = SAN_LIB
    return env


if __name__ == "__main__":
    import sys
    print(build(verbose=True, sanitize="--sanitize" in sys.argv))
