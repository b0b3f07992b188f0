"""Recurrent decode step through the C ABI against the fp64 oracle, alone and as the
continuation of a prefill by ssd_forward (the oracle runs the whole sequence in one
pass, so this also checks that splitting a sequence at any token changes nothing)."""
import numpy as np
import pytest
import torch

from gpu_common import SSM_MAX_TOL_FP32, SSM_RMS_TOL, TOL, dev, needs_gpu, np64
from metrics import max_rel_rms, rms_rel
import oracle
from state_space_sequence_chunk_amd import inputs as gen
from state_space_sequence_chunk_amd import ssd

pytestmark = [pytest.mark.gpu, needs_gpu]


def _print(msg):
    print(msg, flush=True)


def _draw(batch, seqlen, nheads, P, S, G, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return gen.draw(batch, seqlen, nheads, P, S, G, gen.torch_dtype(dtype), g, random_h0=True)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("batch,nheads,P,S,G", [
    (2, 24, 64, 64, 1), (1, 80, 64, 128, 1), (1, 16, 64, 256, 8), (3, 4, 16, 16, 2),
    (2, 6, 128, 32, 3), (1, 2, 32, 256, 1)])
def test_decode_step_matches_oracle(batch, nheads, P, S, G, dtype):
    cpu = _draw(batch, 1, nheads, P, S, G, dtype, 500 + P + S)
    for D in ("given", None):
        Dv = cpu["D"] if D == "given" else None
        ref = oracle.forward(cpu["x"], cpu["dt"], cpu["A"], cpu["B"], cpu["C"], Dv, cpu["h0"])
        state = dev(cpu["h0"]).clone()
        y = ssd.decode_step(dev(cpu["x"][:, 0]), dev(cpu["dt"][:, 0]), dev(cpu["A"]),
                            dev(cpu["B"][:, 0]), dev(cpu["C"][:, 0]), dev(Dv), state)
        torch.cuda.synchronize()
        ey = max_rel_rms(np64(y), ref["y"][:, 0])
        es = max_rel_rms(np64(state), ref["final"])
        _print(f"decode b{batch} H{nheads} P{P} S{S} G{G} {dtype} D={D}: y {ey:.2e} state {es:.2e}")
        # one fp32 step on exactly rounded inputs: far inside either dtype's bound
        assert ey <= 1e-5 and es <= 1e-5


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_prefill_then_decode_equals_one_pass(dtype):
    batch, L1, K, H, P, S, G, T = 2, 256, 12, 8, 64, 128, 2, 64
    cpu = _draw(batch, L1 + K, H, P, S, G, dtype, 77)
    ref = oracle.forward(cpu["x"], cpu["dt"], cpu["A"], cpu["B"], cpu["C"], cpu["D"], cpu["h0"])
    refd = oracle.forward(cpu["x"], cpu["dt"], cpu["A"], cpu["B"], cpu["C"], None, cpu["h0"])
    d = {k: dev(v) for k, v in cpu.items()}
    for Dv, r in ((d["D"], ref), (None, refd)):
        y1, state = ssd.forward(d["x"][:, :L1].contiguous(), d["dt"][:, :L1].contiguous(), d["A"],
                                d["B"][:, :L1].contiguous(), d["C"][:, :L1].contiguous(), Dv,
                                d["h0"], chunk=T)
        ys = [y1]
        for t in range(L1, L1 + K):
            yt = ssd.decode_step(d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                                 d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), Dv, state)
            ys.append(yt[:, None])
        y = torch.cat(ys, dim=1)
        torch.cuda.synchronize()
        ey = max_rel_rms(np64(y), r["y"])
        ed = max_rel_rms(np64(y[:, L1:]), r["y"][:, L1:])
        es = max_rel_rms(np64(state), r["final"])
        _print(f"prefill {L1} + decode {K} {dtype} D={'given' if Dv is not None else 'none'}: "
               f"y {ey:.2e} decoded y {ed:.2e} final {es:.2e}")
        assert ed <= TOL[dtype] and es <= TOL[dtype]
        if Dv is not None:
            assert ey <= TOL[dtype]
        else:  # the SSM path alone: the same gates as the forward pass's D = 0 output
            assert rms_rel(np64(y), r["y"]) <= SSM_RMS_TOL[dtype]
            if dtype == "fp32":
                assert ey <= SSM_MAX_TOL_FP32


def test_decode_is_deterministic_and_in_place():
    cpu = _draw(2, 1, 24, 64, 64, 1, "bf16", 9)
    args = [dev(cpu["x"][:, 0]), dev(cpu["dt"][:, 0]), dev(cpu["A"]), dev(cpu["B"][:, 0]),
            dev(cpu["C"][:, 0]), dev(cpu["D"])]
    s1 = dev(cpu["h0"]).clone()
    s2 = dev(cpu["h0"]).clone()
    p1 = s1.data_ptr()
    y1 = ssd.decode_step(*args, s1)
    y2 = ssd.decode_step(*args, s2)
    torch.cuda.synchronize()
    assert s1.data_ptr() == p1
    assert torch.equal(s1, s2) and torch.equal(y1, y2)
    assert not torch.equal(s1, dev(cpu["h0"]))
