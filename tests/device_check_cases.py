"""Cases for the device-check build of the library (not collected by pytest).

``run(gl)`` runs a set of small seeded launches through the library the binding has
loaded -- the bf16 forward (both forward schedules, split tails), dgrad, the fused
wgrad + bias grad into an fp32 main_grad (contraction plan), the MXFP8 forward and
the grouped MXFP8 quantizer both ways -- and returns their outputs and workspace
status words as CPU tensors.  ``run_tampered(gl)`` runs the bf16 forward on a
workspace whose offsets were changed after the offsets call so that group 0's
second row tile lies past its rows; only the device-check build may run it (its
forward flags the tile and skips it; every access stays inside the buffers either
way, group 1 reading rows 200 .. 455).

As a script (``python tests/device_check_cases.py OUT``, with GL_LIBRARY_PATH naming
the device-check build) it runs both and saves the results to OUT with torch.save.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch

DEV = "cuda"
BF = torch.bfloat16


def _inputs(seed, G, K, N, m):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(m))
    x = torch.randn(T, K, generator=g).to(BF)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(BF)
    b = (torch.randn(G, N, generator=g) * 0.1).to(BF)
    dy = torch.randn(T, N, generator=g).to(BF)
    mg = torch.randn(G, N, K, generator=g)
    return [t.to(DEV) for t in (x, w, b, dy, mg)]


def _workspace(gl, m):
    ws = gl.new_workspace(len(m), torch.device(DEV))
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), int(sum(m)), ws)
    return ws


def run(gl):
    out = {}
    # bf16: small groups (deeper weight ring; every tile split), then large ones
    for name, (G, K, N, m) in {"small": (5, 200, 264, [0, 300, 1, 0, 513]),
                               "large": (2, 200, 264, [700, 301])}.items():
        x, w, b, dy, mg = _inputs(7, G, K, N, m)
        T = int(sum(m))
        ws = _workspace(gl, m)
        y = torch.empty(T, N, dtype=BF, device=DEV)
        gl.gl_forward(x, w, y, ws, bias=b)
        dx = torch.empty(T, K, dtype=BF, device=DEV)
        gl.gl_dgrad(dy, w, dx, ws)
        db = torch.empty(G, N, dtype=BF, device=DEV)
        gl.gl_wgrad_bgrad(x, dy, mg, db, ws, accumulate=True)
        out.update({f"{name}_y": y, f"{name}_dx": dx, f"{name}_main_grad": mg, f"{name}_db": db,
                    f"{name}_status": torch.tensor(gl.gl_read_status(ws))})
    # MXFP8: quantize x and w rowwise, forward; dy both ways in one pass
    G, K, N, m = 3, 256, 256, [0, 300, 77]
    x, w, _, dy, _ = _inputs(11, G, K, N, m)
    T = int(sum(m))
    ws = _workspace(gl, m)
    u8 = dict(dtype=torch.uint8, device=DEV)
    xq, xs = torch.empty(T, K, **u8), torch.empty(T, K // 32, **u8)
    wq, wsc = torch.empty(G, N, K, **u8), torch.empty(G, N, K // 32, **u8)
    gl.gl_group_quantize_mxfp8(x, xq, xs)
    gl.gl_group_quantize_mxfp8(w, wq, wsc)
    y = torch.empty(T, N, dtype=BF, device=DEV)
    gl.gl_forward(xq, wq, y, ws, x_scale=xs, w_scale=wsc)
    ld = gl.gl_colwise_ld(G, T)
    dq, ds = torch.empty(T, N, **u8), torch.empty(T, N // 32, **u8)
    dtq, dts = torch.zeros(N, ld, **u8), torch.zeros(N, ld // 32, **u8)
    gl.gl_group_quantize_mxfp8_rowwise_colwise(dy, dq, ds, dtq, dts, ws, G)
    out.update({"mx_y": y, "mx_dy_rowwise": dq, "mx_dy_rowwise_scale": ds, "mx_dy_colwise": dtq,
                "mx_dy_colwise_scale": dts, "mx_status": torch.tensor(gl.gl_read_status(ws))})
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in out.items()}


def run_tampered(gl):
    G, K, N, m = 4, 128, 264, [300, 200, 0, 100]
    x, w, b, _, _ = _inputs(3, G, K, N, m)
    T = int(sum(m))
    ws = _workspace(gl, m)
    y_ok = torch.empty(T, N, dtype=BF, device=DEV)
    gl.gl_forward(x, w, y_ok, ws, bias=b)
    status_ok = gl.gl_read_status(ws)
    offs = gl.workspace_offsets(ws, G)
    offs[1] = 200  # group 0 keeps its two row tiles in the tile table but now ends at row 200
    y = torch.full((T, N), float("nan"), dtype=BF, device=DEV)
    gl.gl_forward(x, w, y, ws, bias=b)
    status = gl.gl_read_status(ws)
    torch.cuda.synchronize()
    return {"tamper_y_ok": y_ok.cpu(), "tamper_status_ok": torch.tensor(status_ok), "tamper_y": y.cpu(),
            "tamper_status": torch.tensor(status), "tamper_x": x.cpu(), "tamper_w": w.cpu(), "tamper_b": b.cpu()}


if __name__ == "__main__":
    import grouped_gemm_gl_amd as gl

    gl.load()
    print(f"device-check cases on {gl.library_path}", flush=True)
    res = run(gl)
    print("valid cases done", flush=True)
    res.update(run_tampered(gl))
    print("tampered workspace case done", flush=True)
    res["library"] = torch.tensor(list(gl.library_path.encode()), dtype=torch.uint8)
    torch.save(res, sys.argv[1])
