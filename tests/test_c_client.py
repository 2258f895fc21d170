"""The C ABI used from plain C: include/w4a4.h compiles as strict C99 and C++17, and a
C99 program (tests/c/w4a4_c_client.c, hipMalloc'd buffers, no Python or torch) gets
the same host-side answers and, on the GPU, the same s, O and Y bit for bit as the
Python binding on the same inputs."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from bit_quantized_dit_amd import synth
from bit_quantized_dit_amd import w4a4 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "w4a4_c_client.c")
OUT_DIR = os.path.join(ROOT, "tests", "c", "_build")
CLIENT = os.path.join(OUT_DIR, "w4a4_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
LIB_DIR = os.path.dirname(B.LIB_PATH)


def _gcc():
    g = shutil.which("gcc")
    if g is None:
        pytest.skip("gcc not installed")
    return g


def build_client() -> str:
    """Compile the C client (strict C99, warnings as errors) against the in-tree library."""
    os.makedirs(OUT_DIR, exist_ok=True)
    if os.path.exists(CLIENT) and os.path.getmtime(CLIENT) >= max(os.path.getmtime(SRC), os.path.getmtime(B.LIB_PATH)):
        return CLIENT
    cmd = [_gcc(), "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"), SRC,
           "-L", LIB_DIR, "-lw4a4", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{LIB_DIR}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", CLIENT + ".tmp"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(CLIENT + ".tmp", CLIENT)
    return CLIENT


@pytest.mark.parametrize("std,lang", [("c99", "c"), ("c11", "c"), ("c++17", "c++")])
def test_header_compiles_strict(std, lang):
    """The public header alone, with no other include, under -pedantic -Werror."""
    src = '#include "w4a4.h"\nint main(void) { w4a4_packed d; (void)d; return W4A4_OK; }\n'
    cmd = [_gcc() if lang == "c" else shutil.which("g++"), f"-std={std}", "-Wall", "-Wextra", "-Werror",
           "-pedantic", "-fsyntax-only", "-x", lang, "-I", os.path.join(ROOT, "include"), "-"]
    r = subprocess.run(cmd, input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_client_host_queries():
    out = subprocess.run([build_client(), "host"], check=True, capture_output=True, text=True).stdout
    vals = dict(line.split(" ", 1) for line in out.strip().split("\n") if not line.startswith("status"))
    assert int(vals["packed_size"]) == B.w4a4_packed_size(512, 1024, 16, 0)
    assert int(vals["packed_size_bad_k"]) == 1
    names = [line.split(" ", 2)[2] for line in out.strip().split("\n") if line.startswith("status")]
    assert names == [B.status_string(s) for s in range(6)]


@pytest.mark.gpu
def test_c_client_matches_binding():
    import torch

    client = build_client()
    spec = synth.WORKLOADS[1]
    T, d_in, d_out, k, layout, T_cal = 200, 512, 320, 16, 0, 128
    inp = synth.layer_inputs(spec, T=T, d_in=d_in, d_out=d_out, k=k, T_cal=T_cal)
    X, Xc, W = (np.ascontiguousarray(inp[n], dtype=np.float32) for n in ("X", "X_cal", "W"))
    fin, fout = os.path.join(OUT_DIR, "c_client_in.bin"), os.path.join(OUT_DIR, "c_client_out.bin")
    with open(fin, "wb") as f:
        f.write(np.array([T, d_in, d_out, k, layout, T_cal], dtype=np.int64).tobytes())
        f.write(np.array([spec.alpha], dtype=np.float32).tobytes())
        f.write(X.tobytes() + Xc.tobytes() + W.tobytes())
    r = subprocess.run([client, "run", fin, fout], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(fout, "rb").read()
    s_c = np.frombuffer(raw, np.float32, d_in)
    O_c = np.frombuffer(raw, np.int32, k, offset=4 * d_in)
    Y_c = np.frombuffer(raw, np.float32, T * d_out, offset=4 * (d_in + k)).reshape(T, d_out)
    # the same calls through the Python binding
    s, O, _, _ = B.w4a4_calibrate_scales(torch.from_numpy(Xc).cuda(), torch.from_numpy(W).cuda(), spec.alpha, k)
    packed = B.w4a4_pack_weights(torch.from_numpy(W).cuda(), s, O, layout)
    ws = B.alloc_workspace(T, packed)
    Y = torch.empty(T, d_out, dtype=torch.float32, device="cuda")
    B.w4a4_linear(torch.from_numpy(X).cuda(), packed, Y, ws)
    torch.cuda.synchronize()
    assert np.array_equal(s_c.view(np.uint32), s.view(np.uint32))
    assert np.array_equal(O_c, O)
    assert np.array_equal(Y_c.view(np.uint32), Y.cpu().numpy().view(np.uint32))
