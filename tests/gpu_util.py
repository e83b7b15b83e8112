"""Shared helpers of the GPU parity tests (device, library, conversions, tolerances)."""
import numpy as np

REL_FRO = 5e-3      # ||G-R||_F / ||R||_F
REL_MAX = 2e-2      # max|G-R| / max|R|


def gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("these tests need an MI355X GPU")
    import bit_quantized_moe_amd as bqm
    bqm.load()                       # fails loudly if libbqm.so is missing
    return torch.device("cuda")


def np_f32(t):
    return t.detach().float().cpu().numpy()


def np_u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def assert_close(got, ref, name, rel_fro=REL_FRO, rel_max=REL_MAX):
    from oracle.moe import rel_errors
    fro, mx = rel_errors(got, ref)
    assert fro <= rel_fro and mx <= rel_max, f"{name}: rel_fro={fro:.3e} rel_max={mx:.3e}"
    return fro, mx


def log(msg):
    print(msg, flush=True)
