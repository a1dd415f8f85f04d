"""mhla_forward_noalloc (the entry point for callers that cannot allocate
device memory) against mhla_forward_ex, through the C ABI: the same kernels,
so the outputs must be bit-identical.  Two calls in a row on one device, the
second with a smaller input, for each path that uses scratch; a call whose
scratch need exceeds the fixed array is rejected before any launch."""
import numpy as np
import pytest
import torch

import token_level_head_mhla_amd as m
from mhla_inputs import DTYPE_BF16, DTYPE_F32, PHI_ELU1, PHI_RELU, WORKLOADS, custom_workload, make_inputs
from gpu_util import to_device

pytestmark = pytest.mark.gpu


def _both(inp, path=m.MHLA_PATH_AUTO):
    wl = inp.wl
    dev = to_device(inp)
    ref = torch.empty_like(dev[0])
    out = torch.full_like(dev[0], float("nan"))
    m.mhla_forward_ex(*dev, ref, (wl.grid, wl.block), wl.phi, wl.flags, path)
    m.mhla_forward_noalloc(*dev, out, (wl.grid, wl.block), wl.phi, wl.flags, path)
    torch.cuda.synchronize()
    need = m.mhla_workspace_bytes_ex(wl.B, wl.H, wl.N, wl.d, m.BlockShape.make(wl.grid, wl.block),
                                     wl.dtype, wl.flags, path)
    return ref, out, need


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.parametrize("first,second", [
    # blocked path: the 4096-token image shape, then one batch item of it
    (("hires", 4), ("hires", 1)),
    # large-M mixing (coefficients in the scratch too): video-latent, then a
    # 256-block shape
    (("video", 1), ("m256", 2)),
    # chunkwise causal form, then a smaller causal call
    (("lm_causal", 16), ("lm_causal", 3)),
    # fp32 generic path in its three-kernel form (fp32 tables), then a smaller
    # fp32 call (slices too large for the single-launch form)
    (("f32_256", 1), ("f32_128", 1)),
])
def test_noalloc_matches_the_allocating_entry_point(first, second):
    shapes = {
        "m256": custom_workload(2, 2, 64, (4, 32, 32), (1, 4, 4), PHI_ELU1, DTYPE_BF16, index=41),
        "f32_256": custom_workload(1, 2, 64, (1, 16, 16), (1, 4, 4), PHI_RELU, DTYPE_F32,
                                   index=42),
        "f32_128": custom_workload(1, 1, 64, (1, 8, 16), (1, 4, 4), PHI_ELU1, DTYPE_F32,
                                   index=43),
    }
    sizes = []
    for name, B in (first, second):
        wl = shapes.get(name) or WORKLOADS[name]
        inp = make_inputs(wl, B=B if name in WORKLOADS else None)
        ref, out, need = _both(inp)
        print("NOALLOC %s B=%d scratch=%d bytes" % (name, inp.wl.B, need))
        assert 0 < need <= m.MHLA_NOALLOC_SCRATCH_BYTES
        assert _same(out, ref)
        sizes.append(need)
    assert sizes[1] < sizes[0]


def test_noalloc_paths_without_scratch():
    """The fused and token-pair paths, and the generic path's single-launch
    form (the tiny fp32 problem), keep everything on chip."""
    for name in ("deit_t", "dit_xl2", "tiny"):
        inp = make_inputs(WORKLOADS[name], B=2)
        ref, out, need = _both(inp)
        assert need == 0
        assert _same(out, ref)


def test_noalloc_rejects_calls_beyond_the_scratch():
    """16 batch items of the 4096-token image need about 277 MB of scratch."""
    wl = WORKLOADS["hires"]
    need = m.mhla_workspace_bytes(16, wl.H, wl.N, wl.d, m.BlockShape.make(wl.grid, wl.block),
                                  wl.dtype)
    assert need > m.MHLA_NOALLOC_SCRATCH_BYTES
    shape = (16, wl.H, wl.N, wl.d)
    q = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    w = torch.full((wl.H, wl.M, wl.M), 1.0 / wl.M, dtype=torch.float32, device="cuda")
    out = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MhlaError) as ei:
        m.mhla_forward_noalloc(q, q, q, w, out, (wl.grid, wl.block), wl.phi)
    assert ei.value.code == m.MHLA_ERR_UNSUPPORTED
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
