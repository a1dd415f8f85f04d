"""GPU parity of incremental (streaming) inference: mhla_decode_step called
token by token (and mhla_decode_steps over several tokens a call,
mhla_decode_prefill from a prompt) through the C ABI against the oracle's token-by-token causal
inference (MHLA paper App. C), which is pinned to the chunkwise causal forward.

Gate: max over (batch, head) slices of max|y - y_oracle| / max|y_oracle| over
the whole sequence, 1e-5 for fp32 and 1e-2 for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import token_level_head_mhla_amd as m
from mhla_inputs import (DTYPE_BF16, DTYPE_F32, FLAG_CAUSAL, FLAG_NO_NORM, PHI_ELU1, PHI_RELU,
                         custom_workload, make_inputs)
from gpu_util import TOL, slice_error, to_device, to_f64

pytestmark = pytest.mark.gpu


def _stream(inp, nb, flags=0):
    """Feed the sequence one token at a time; returns Y [B, H, N, d] on the host."""
    wl = inp.wl
    q, k, v, w = to_device(inp)
    B, H, N, d = q.shape
    M = N // nb
    qt, kt, vt = (x.permute(2, 0, 1, 3).contiguous() for x in (q, k, v))   # [N, B, H, d]
    state = torch.empty(m.mhla_decode_state_bytes(B, H, d, M) // 4, dtype=torch.float32,
                        device="cuda")
    state.fill_(float("nan"))   # the first token of every chunk must not read stale state
    y = torch.empty_like(qt)
    for t in range(N):
        m.mhla_decode_step(qt[t], kt[t], vt[t], w, y[t], state, M, nb, t, wl.phi, flags)
    torch.cuda.synchronize()
    return to_f64(y.permute(1, 2, 0, 3).contiguous())


DECODE_CASES = [
    # (B, H, N, nb, d, phi, dtype)
    (2, 3, 256, 64, 64, PHI_ELU1, DTYPE_BF16),    # the LM chunk size, 4 chunks
    (1, 2, 96, 16, 72, PHI_RELU, DTYPE_BF16),
    (2, 2, 40, 1, 32, PHI_ELU1, DTYPE_BF16),      # a chunk per token
    (1, 2, 48, 48, 16, PHI_ELU1, DTYPE_BF16),     # a single chunk
    (1, 1, 64, 16, 16, PHI_RELU, DTYPE_F32),
    (1, 2, 32, 8, 128, PHI_ELU1, DTYPE_F32),      # d = 128: LDS above 64 KB
    (1, 2, 30, 6, 13, PHI_ELU1, DTYPE_F32),       # odd d in fp32
]


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("B,H,N,nb,d,phi,dtype", DECODE_CASES)
def test_decode_stream(B, H, N, nb, d, phi, dtype, norm):
    flags = FLAG_CAUSAL | (0 if norm else FLAG_NO_NORM)
    wl = custom_workload(B, H, d, (1, 1, N), (1, 1, nb), phi, dtype,
                         index=hash((N, nb, d)) % 937, flags=flags)
    inp = make_inputs(wl)
    y = _stream(inp, nb, flags)
    ref = oracle.np_decode(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, nb, phi, norm=norm)
    err = slice_error(y, ref)
    print("PARITY decode N=%d nb=%d d=%d phi=%d dtype=%d norm=%d err=%.3e"
          % (N, nb, d, phi, dtype, norm, err))
    assert np.all(np.isfinite(y))
    assert err <= TOL[dtype]


def test_decode_matches_chunkwise_forward_on_gpu():
    """The streamed outputs and the chunkwise causal forward (blocked path) of
    the same inputs agree to the bf16 gate."""
    wl = custom_workload(2, 2, 64, (1, 1, 256), (1, 1, 64), PHI_ELU1, DTYPE_BF16, index=41,
                         flags=FLAG_CAUSAL | FLAG_NO_NORM)
    inp = make_inputs(wl)
    y_dec = _stream(inp, 64, wl.flags)
    q, k, v, w = to_device(inp)
    out = torch.empty_like(q)
    m.mhla_forward_ex(q, k, v, w, out, (wl.grid, wl.block), wl.phi, wl.flags)
    torch.cuda.synchronize()
    err = slice_error(y_dec, to_f64(out))
    print("PARITY decode vs chunkwise forward err=%.3e" % err)
    assert err <= TOL[DTYPE_BF16]


PREFILL_CASES = [
    # (B, H, N, nb, d, phi, dtype, T): T prompt tokens, then decoding to N
    (2, 3, 256, 64, 64, PHI_ELU1, DTYPE_BF16, 100),   # the prompt ends inside chunk 1
    (2, 3, 256, 64, 64, PHI_ELU1, DTYPE_BF16, 128),   # ... on a chunk boundary
    (1, 2, 96, 16, 72, PHI_RELU, DTYPE_BF16, 1),      # a one-token prompt
    (1, 1, 64, 16, 16, PHI_RELU, DTYPE_F32, 63),
    (1, 2, 32, 8, 128, PHI_ELU1, DTYPE_F32, 20),      # d = 128
    (1, 2, 30, 6, 13, PHI_ELU1, DTYPE_F32, 30),       # odd d; the whole sequence as prompt
]


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("B,H,N,nb,d,phi,dtype,T", PREFILL_CASES)
def test_decode_prefill(B, H, N, nb, d, phi, dtype, T, norm):
    """mhla_decode_prefill leaves the state of T decode steps, bit for bit, and
    decoding continues from it to the oracle's outputs."""
    flags = FLAG_CAUSAL | (0 if norm else FLAG_NO_NORM)
    wl = custom_workload(B, H, d, (1, 1, N), (1, 1, nb), phi, dtype,
                         index=hash((N, nb, d, T)) % 911, flags=flags)
    inp = make_inputs(wl)
    q, k, v, w = to_device(inp)
    M = N // nb
    qt, kt, vt = (x.permute(2, 0, 1, 3).contiguous() for x in (q, k, v))   # [N, B, H, d]
    words = m.mhla_decode_state_bytes(B, H, d, M) // 4
    stepped = torch.full((words,), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.empty_like(qt)
    for t in range(T):
        m.mhla_decode_step(qt[t], kt[t], vt[t], w, y[t], stepped, M, nb, t, wl.phi, flags)
    filled = torch.full((words,), float("nan"), dtype=torch.float32, device="cuda")
    m.mhla_decode_prefill(k[:, :, :T].contiguous(), v[:, :, :T].contiguous(), w, filled, M, nb,
                          wl.phi, flags)
    torch.cuda.synchronize()
    assert torch.equal(stepped.view(torch.int32), filled.view(torch.int32))
    for t in range(T, N):
        m.mhla_decode_step(qt[t], kt[t], vt[t], w, y[t], filled, M, nb, t, wl.phi, flags)
    torch.cuda.synchronize()
    if T == N:
        return
    got = to_f64(y.permute(1, 2, 0, 3).contiguous())[:, :, T:]
    ref = oracle.np_decode(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, nb, phi, norm=norm)[:, :, T:]
    err = slice_error(got, ref)
    print("PARITY decode prefill N=%d nb=%d d=%d T=%d dtype=%d norm=%d err=%.3e"
          % (N, nb, d, T, dtype, norm, err))
    assert err <= TOL[dtype]


STEPS_CASES = [
    # (B, H, N, nb, d, phi, dtype, sizes): tokens per call, cycled until N
    (2, 3, 256, 64, 64, PHI_ELU1, DTYPE_BF16, (1, 3, 64, 133, 7)),   # calls across chunk ends
    (2, 3, 256, 64, 64, PHI_ELU1, DTYPE_BF16, (256,)),               # the whole sequence at once
    (1, 2, 96, 16, 72, PHI_RELU, DTYPE_BF16, (16,)),                 # calls on chunk boundaries
    (1, 1, 64, 16, 16, PHI_RELU, DTYPE_F32, (5, 1, 40)),
    (1, 2, 32, 8, 128, PHI_ELU1, DTYPE_F32, (9, 2)),                 # d = 128
    (1, 2, 30, 6, 13, PHI_ELU1, DTYPE_F32, (4, 11)),                 # odd d
]


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("B,H,N,nb,d,phi,dtype,sizes", STEPS_CASES)
def test_decode_steps(B, H, N, nb, d, phi, dtype, sizes, norm):
    """mhla_decode_steps over calls of several tokens leaves the outputs and the
    state of one mhla_decode_step per token, bit for bit, and the outputs
    match the oracle."""
    flags = FLAG_CAUSAL | (0 if norm else FLAG_NO_NORM)
    wl = custom_workload(B, H, d, (1, 1, N), (1, 1, nb), phi, dtype,
                         index=hash((N, nb, d, sizes)) % 907, flags=flags)
    inp = make_inputs(wl)
    q, k, v, w = to_device(inp)
    M = N // nb
    qt, kt, vt = (x.permute(2, 0, 1, 3).contiguous() for x in (q, k, v))   # [N, B, H, d]
    words = m.mhla_decode_state_bytes(B, H, d, M) // 4
    stepped = torch.full((words,), float("nan"), dtype=torch.float32, device="cuda")
    y1 = torch.empty_like(qt)
    for t in range(N):
        m.mhla_decode_step(qt[t], kt[t], vt[t], w, y1[t], stepped, M, nb, t, wl.phi, flags)
    grouped = torch.full((words,), float("nan"), dtype=torch.float32, device="cuda")
    yn = torch.full_like(q, float("nan"))
    t0, c = 0, 0
    while t0 < N:
        n = min(sizes[c % len(sizes)], N - t0)
        part = torch.empty_like(q[:, :, t0:t0 + n])
        m.mhla_decode_steps(q[:, :, t0:t0 + n].contiguous(), k[:, :, t0:t0 + n].contiguous(),
                            v[:, :, t0:t0 + n].contiguous(), w, part, grouped, M, nb, t0,
                            wl.phi, flags)
        yn[:, :, t0:t0 + n] = part
        t0, c = t0 + n, c + 1
    torch.cuda.synchronize()
    assert torch.equal(stepped.view(torch.int32), grouped.view(torch.int32))
    y1 = y1.permute(1, 2, 0, 3).contiguous()
    assert torch.equal(y1.view(torch.int16 if dtype == DTYPE_BF16 else torch.int32),
                       yn.view(torch.int16 if dtype == DTYPE_BF16 else torch.int32))
    ref = oracle.np_decode(inp.q_f64, inp.k_f64, inp.v_f64, inp.w_f64, nb, phi, norm=norm)
    err = slice_error(to_f64(yn), ref)
    print("PARITY decode steps N=%d nb=%d d=%d sizes=%s dtype=%d norm=%d err=%.3e"
          % (N, nb, d, sizes, dtype, norm, err))
    assert err <= TOL[dtype]
