"""Helpers for the GPU parity tests: device transfer and the two sides' inputs.

Both sides start from the same seeded draws (``synth``): the HIP path quantises
and packs with the library's own host routines, the oracle with its own code.
"""

import numpy as np

import oracle


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible HIP device")
    return torch


def dev(a: np.ndarray):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def gaussian_sides(lib, w: np.ndarray, group: int):
    """(packed, scales) from the library and (packed_ref, scales_ref) from the oracle."""
    packed, scales = lib.quantize(w, group)
    q_ref, s_ref = oracle.quantize(w, group)
    p_ref = oracle.pack(q_ref)
    return (packed, scales), (p_ref, s_ref)


def assert_close(y_gpu, y_ref, what=""):
    rep = oracle.compare(y_gpu, y_ref)
    assert rep.ok, f"{what}: {rep.message}"
    return rep


def assert_bit_exact(y_gpu: np.ndarray, y_ref: np.ndarray, what=""):
    """The GPU output must be the fp16 rounding (nearest even) of the exact result.

    Holds when every partial sum is exact in fp32, which the integer family
    guarantees by construction (small integers times powers of two spanning a
    few octaves); checked here on the final value as a precondition.
    """
    assert np.array_equal(y_ref.astype(np.float32).astype(np.float64), y_ref), f"{what}: reference not exact in fp32"
    want = y_ref.astype(np.float16)
    bad = np.argwhere(y_gpu.view(np.uint16) != want.view(np.uint16))
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: " \
                          f"got {y_gpu[tuple(bad[0])]!r} want {want[tuple(bad[0])]!r}"
