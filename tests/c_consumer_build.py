"""Compiles tests/c_consumer.c, a plain C program that links libfrattn and the
HIP runtime only (no framework types)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_consumer(out_path):
    from gqa_decode_attention_fr_amd import binding
    libdir = os.path.dirname(binding.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROCM, 'include')}",
           os.path.join(HERE, "c_consumer.c"), f"-L{libdir}", "-lfrattn",
           f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{libdir}",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(out_path)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out_path
