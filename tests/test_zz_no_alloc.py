"""ssd_forward_noalloc (the forward pass in the library's own per-device scratch array)
against ssd_forward, through the C ABI: two calls in a row, the second on a smaller
problem (the array keeps the first call's contents), each bitwise equal to ssd_forward on
the same inputs, and the small one also within the parity bound of the fp64 oracle."""
import pytest
import torch

from gpu_common import TOL, make, needs_gpu, oracle_forward
from metrics import max_rel_rms
from state_space_sequence_chunk_amd import inputs as gen
from state_space_sequence_chunk_amd import ssd

pytestmark = [pytest.mark.gpu, needs_gpu]


def _both(w):
    cpu, d = make(w)
    f = ssd.Forward(d["x"], d["B"], w.chunk)
    y_ref, fin_ref = f(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    torch.cuda.synchronize()
    y_ref, fin_ref = y_ref.clone(), fin_ref.clone()
    del f
    y = torch.full_like(y_ref, float("nan"))
    fin = torch.full_like(fin_ref, float("nan"))
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    ssd.ssd_forward_noalloc(sh, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], y, fin)
    torch.cuda.synchronize()
    return cpu, y, fin, y_ref, fin_ref


def test_noalloc_equals_forward_large_then_small():
    large = gen.WORKLOADS["2.7b-bf16"]
    sh = ssd.make_shape(large.batch, large.seqlen, large.nheads, large.headdim, large.dstate,
                        large.ngroups, large.chunk, torch.bfloat16)
    need = ssd.forward_workspace_bytes(sh)
    print(f"2.7b-bf16: forward workspace {need} of {ssd.NOALLOC_SCRATCH_BYTES} bytes", flush=True)
    assert need <= ssd.NOALLOC_SCRATCH_BYTES
    for w in (large, gen.WORKLOADS["small-bf16"], gen.WORKLOADS["small-fp32"]):
        cpu, y, fin, y_ref, fin_ref = _both(w)
        same = bool(torch.equal(y, y_ref)) and bool(torch.equal(fin, fin_ref))
        print(f"{w.name}: noalloc bitwise equal to ssd_forward: {same}", flush=True)
        assert same
        if w.seqlen * w.batch <= 4096:
            ref = oracle_forward(cpu)
            ey, ef = max_rel_rms(y, ref["y"]), max_rel_rms(fin, ref["final"])
            print(f"{w.name}: y max/rms {ey:.2e} final max/rms {ef:.2e}", flush=True)
            assert ey <= TOL[w.dtype] and ef <= TOL[w.dtype]
        del y, fin, y_ref, fin_ref
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_problem_past_its_scratch():
    w = gen.WORKLOADS["long-bf16"]
    cpu, d = make(w)
    sh = ssd.shape_of(d["x"], d["B"], w.chunk)
    assert ssd.forward_workspace_bytes(sh) > ssd.NOALLOC_SCRATCH_BYTES
    y = torch.empty(d["x"].shape, dtype=torch.float32, device="cuda")
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_forward_noalloc(sh, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], y,
                                None)
    assert e.value.code == 8
