"""Helpers shared by the GPU parity tests: device transfer and the parity metric."""
import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-5}


def torch_dtype(name):
    import torch

    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def dev(a, dtype="bf16"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0").to(torch_dtype(dtype))


def host(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy()


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    scale = np.abs(ref).max()
    if scale == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / scale)


def assert_close(name, got, ref, tol):
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    e = rel_err(got, ref)
    print(f"  {name:8s} max|err|/max|ref| = {e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: max|err|/max|ref| = {e:.3e} > {tol:g}"


def proj_dev(p, dtype="bf16", nf4=None, adapters=None):
    """Device projection; ``adapters="f32"`` keeps A and B in fp32 (the fp32
    LoRA-gradient mode when ``dtype`` is bf16)."""
    import adapter_mlp_amd as lm

    ad = adapters or dtype
    return lm.Proj(A=dev(p["A"], ad), B=dev(p["B"], ad), scale=p["s"],
                   W=None if nf4 is not None else dev(p["W"], dtype), nf4=nf4)
