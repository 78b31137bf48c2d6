"""Builds tests/c_abi_driver.cpp (a C ABI caller with no Python) into
tests/_bin/c_abi_driver, linked against the in-tree libchunkattn.so."""
import os
import subprocess

from kv_cache_attention_chunk_amd import build as pkg

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c_abi_driver.cpp")
OUT = os.path.join(HERE, "_bin", "c_abi_driver")


def build() -> str:
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    rpath = os.path.relpath(pkg.PKG, os.path.dirname(OUT))
    cmd = [pkg.hipcc(), "-O2", "-std=c++17", f"--offload-arch={pkg.ARCH}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", pkg.INCLUDE, SRC, "-L", pkg.PKG, "-lchunkattn",
           f"-Wl,-rpath,$ORIGIN/{rpath}", "-o", OUT + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C ABI driver failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build())
