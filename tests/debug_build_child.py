"""Child process of test_gpu_debug_build.py: runs with MOE_LIB pointing at the MOE_DEBUG
build (range-checked GEMM operand loads, host validation of device index data). Runs a bf16
layer forward and an MXFP8 training step on valid inputs and saves their outputs, then hands
the entry points corrupted index data (the debug build must reject it on the host before
launching anything). Usage: python tests/debug_build_child.py OUT.npz"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import moe_inputs as mi  # noqa: E402
from tests.debug_build_run import run_layer, run_mx_step  # noqa: E402


def main(out):
    from dropless_mixture_experts_device_amd import _lib as L
    assert L._LIB_PATH.endswith("libmoe_debug.so"), L._LIB_PATH
    res = {}
    res.update(run_layer())
    res.update(run_mx_step())
    # corrupted index data: each call must raise with MOE_EINVAL and enqueue nothing
    rejected = []
    w = mi.WORKLOADS["small_sigmoid"]
    G, K, N = 4, 64, 64
    A = torch.zeros((40, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((G, N, K), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((40, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((L.moe_workspace_bytes(L.MOE_OP_GROUPED_GEMM, 0, 0, 0, 0, G),), dtype=torch.uint8, device="cuda")
    cases = {
        "offsets decreasing": (torch.tensor([0, 20, 10, 30, 40], dtype=torch.int32, device="cuda"), None),
        "offsets past M": (torch.tensor([0, 10, 20, 30, 41], dtype=torch.int32, device="cuda"), None),
        "gather index out of range": (torch.tensor([0, 10, 20, 30, 40], dtype=torch.int32, device="cuda"),
                                      torch.full((40,), 40, dtype=torch.int32, device="cuda")),
    }
    for name, (off, ar) in cases.items():
        try:
            L.moe_grouped_gemm(A, B, C, off, L.MOE_EPI_NONE, a_rows=ar, workspace=ws)
        except L.MoeError as e:
            if e.status == L.MOE_EINVAL:
                rejected.append(name)
    T, E, k = 16, 8, 2
    offs = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    row_of = torch.empty((T, k), dtype=torch.int32, device="cuda")
    src = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    pws = torch.empty((L.moe_workspace_bytes(L.MOE_OP_PERMUTE, T, 64, E, k, 0),), dtype=torch.uint8, device="cuda")
    for name, idx in (("expert id out of range", np.full((T, k), E)), ("expert id repeated", np.zeros((T, k)))):
        try:
            L.moe_permute(None, torch.from_numpy(idx.astype(np.int32)).cuda(), E, False, offs, row_of, src, None, pws,
                          d=64)
        except L.MoeError as e:
            if e.status == L.MOE_EINVAL:
                rejected.append(name)
    torch.cuda.synchronize()
    res["rejected"] = np.array(rejected)
    np.savez(out, **res)
    print("debug child ok:", ", ".join(rejected), flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
