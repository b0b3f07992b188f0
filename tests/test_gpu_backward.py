"""Parity of the HIP backward pass (through the C ABI) with the fp64 gradient oracle.

The oracle's gradients are pinned by finite differences on the CPU. Bounds on
max|got - oracle| / rms(oracle) for every gradient: 1e-4 with fp32 inputs (fp32
arithmetic, the longest chains being the per-chunk sums over a chunk's tokens and the
inner products over a head's P x S state), 2e-2 with bf16 inputs (the recomputed
chunk-initial states go through the bf16 forward state pass, as in the forward parity
bound). dA, one number per head, sums dt_t dL/da_t over the sequence; dL/da_t is summed
from the end of its own chunk (anchored there by the inner product of gradient and
state), so its rounding does not grow with the sequence length and dA takes the same
bounds.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import dev, needs_gpu, reduced
from metrics import max_rel_rms
from state_space_sequence_chunk_amd import inputs as gen
from state_space_sequence_chunk_amd import ssd

pytestmark = [pytest.mark.gpu, needs_gpu]

W = gen.WORKLOADS
TOL = {"fp32": 1e-4, "bf16": 2e-2}
NAMES = ("dx", "ddt", "dA", "dB", "dC", "dD", "dh0")


def _print(msg):
    print(msg, flush=True)


def problem(batch, L, H, P, S, G, dtype, seed, h0=True):
    g = torch.Generator()
    g.manual_seed(seed)
    cpu = gen.draw(batch, L, H, P, S, G, gen.torch_dtype(dtype), g, random_h0=h0)
    cpu.update(gen.draw_cotangents(batch, L, H, P, S, g))
    return cpu


def run_gpu(cpu, chunk, *, D=True, h0=True, dfinal=True):
    d = {k: dev(v) for k, v in cpu.items()}
    out = ssd.backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"] if D else None,
                       d["h0"] if h0 else None, d["dy"], d["dfinal"] if dfinal else None,
                       chunk=chunk)
    torch.cuda.synchronize()
    return out


def run_oracle(cpu, *, D=True, h0=True, dfinal=True):
    return oracle.backward(cpu["x"], cpu["dt"], cpu["A"], cpu["B"], cpu["C"],
                           cpu["D"] if D else None, cpu["h0"] if h0 else None, cpu["dy"],
                           cpu["dfinal"] if dfinal else None)


def check(tag, got, ref, dtype, names=NAMES):
    errs = {n: max_rel_rms(got[n], ref[n]) for n in names}
    _print(f"{tag}: " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], f"{tag}: {n} max|d|/rms = {e:.2e} > {TOL[dtype]}"


# The five workloads at sizes the oracle finishes in seconds: the small ones whole, the
# large ones on one batch row, 1024 tokens (several chunks) and their heads per group.
SMALL = {
    "tiny-fp32": W["tiny-fp32"],
    "small-fp32": reduced(W["small-fp32"], seqlen=1024),
    "small-bf16": reduced(W["small-bf16"], seqlen=1024),
    "780m-bf16": reduced(W["780m-bf16"], batch=1, seqlen=1024, nheads=16),
    "2.7b-bf16": reduced(W["2.7b-bf16"], batch=1, seqlen=1024, nheads=20),
    "long-bf16": reduced(W["long-bf16"], batch=1, seqlen=1024, nheads=40),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_parity(name):
    w = SMALL[name]
    cpu = problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype,
                  w.seed, h0=w.h0)
    _print(f"{name}: {w.describe()}")
    check(name, run_gpu(cpu, w.chunk), run_oracle(cpu), w.dtype)


# State shapes whose workgroups span 2 and 4 waves (cross-wave sums through LDS), one
# head per group and shared groups, with a ragged last chunk.
@pytest.mark.parametrize("shape", [
    (1, 200, 2, 128, 256, 1, 64), (2, 130, 4, 64, 256, 2, 64), (1, 330, 2, 128, 128, 2, 128),
    (1, 100, 3, 32, 16, 1, 64), (2, 77, 2, 16, 64, 2, 64)])
def test_backward_state_shapes(shape):
    b, L, H, P, S, G, T = shape
    cpu = problem(b, L, H, P, S, G, "fp32", seed=7 + L)
    check(f"shape {shape}", run_gpu(cpu, T), run_oracle(cpu), "fp32")


@pytest.mark.parametrize("dtype,L,T", [("fp32", 300, 64), ("bf16", 700, 256), ("fp32", 1, 64),
                                       ("bf16", 257, 128), ("fp32", 63, 64)])
def test_backward_ragged(dtype, L, T):
    cpu = problem(2, L, 4, 64, 128, 2, dtype, seed=L)
    check(f"ragged {dtype} L={L} T={T}", run_gpu(cpu, T), run_oracle(cpu), dtype)


@pytest.mark.parametrize("D,h0,dfinal", [(False, True, True), (True, False, True),
                                         (True, True, False), (False, False, False)])
def test_backward_optional_inputs(D, h0, dfinal):
    cpu = problem(1, 200, 4, 64, 64, 1, "fp32", seed=31)
    got = run_gpu(cpu, 64, D=D, h0=h0, dfinal=dfinal)
    check(f"D={D} h0={h0} dfinal={dfinal}", got, run_oracle(cpu, D=D, h0=h0, dfinal=dfinal),
          "fp32")


def test_backward_null_optional_outputs():
    # dD and dh0 are optional outputs; the others are the same as with them
    cpu = problem(1, 150, 2, 32, 32, 1, "fp32", seed=5)
    d = {k: dev(v) for k, v in cpu.items()}
    full = run_gpu(cpu, 64)
    sh = ssd.shape_of(d["x"], d["B"], 64, torch.float32)
    out = {n: torch.full_like(full[n], float("nan")) for n in NAMES}
    ws = torch.empty(ssd.backward_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    ssd.ssd_backward(sh, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], d["dy"],
                     d["dfinal"], out["dx"], out["ddt"], out["dA"], out["dB"], out["dC"], None,
                     None, ws)
    torch.cuda.synchronize()
    for n in ("dx", "ddt", "dA", "dB", "dC"):
        assert torch.equal(out[n], full[n]), n
    assert torch.isnan(out["dD"]).all() and torch.isnan(out["dh0"]).all()


def test_backward_empty_sequence():
    cpu = problem(2, 0, 4, 16, 32, 2, "fp32", seed=3)
    for dfinal in (True, False):
        got = run_gpu(cpu, 64, dfinal=dfinal)
        want = cpu["dfinal"] if dfinal else torch.zeros_like(cpu["dfinal"])
        assert torch.equal(got["dh0"].cpu(), want)
        assert not got["dA"].any() and not got["dD"].any()
        assert got["dx"].numel() == 0 and got["dB"].numel() == 0


def test_backward_full_size_sampled_heads():
    # The 2.7B-shape layer at full size (2 x 16384 tokens, 80 heads sharing one B, C): the
    # oracle on 4 sampled heads, each as its own group with the shared B, C, gives those
    # heads' dx, ddt, dA, dD and dh0 exactly (dB and dC sum over all 80 heads and are
    # covered at reduced size).
    w = W["2.7b-bf16"]
    cpu = problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype,
                  w.seed, h0=True)
    got = run_gpu(cpu, w.chunk)
    heads = [0, 27, 53, 79]
    hs = torch.tensor(heads)
    g_of = hs // (w.nheads // w.ngroups)
    sub = {"x": cpu["x"][:, :, hs], "dt": cpu["dt"][:, :, hs], "A": cpu["A"][hs],
           "B": cpu["B"][:, :, g_of], "C": cpu["C"][:, :, g_of], "D": cpu["D"][hs],
           "h0": cpu["h0"][:, hs], "dy": cpu["dy"][:, :, hs], "dfinal": cpu["dfinal"][:, hs]}
    ref = run_oracle(sub)
    got_s = {"dx": got["dx"][:, :, heads], "ddt": got["ddt"][:, :, heads],
             "dA": got["dA"][heads], "dD": got["dD"][heads], "dh0": got["dh0"][:, heads]}
    check("2.7b-bf16 full size, heads " + str(heads), got_s, ref, "bf16",
          names=("dx", "ddt", "dA", "dD", "dh0"))


@pytest.mark.parametrize("name", ["780m-bf16", "2.7b-bf16"])
def test_backward_full_size_all_elements(name):
    # Every element of every gradient at full size against the oracle (a few seconds on the
    # host's threads). The shapes take the matrix-core kernels with their full plans: the
    # per-chunk gradient sums over blocks of heads (12 at the 780M shape, 40 at 2.7B), and
    # at 780M the heads of a group split over two workgroups (dB, dC summed afterwards).
    w = W[name]
    cpu = problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype,
                  w.seed, h0=True)
    got = run_gpu(cpu, w.chunk)
    got = {n: v.cpu() for n, v in got.items()}
    ref = run_oracle(cpu)
    check(name + " full size, all elements", got, ref, "bf16")


def test_backward_long_full_size_sampled_heads():
    # The long workload at full size (65536 tokens, 80 heads in 8 groups): the matrix-core
    # plan runs at 64-token chunks, whose fp32 chunk states (5.4 GB for the batch row) pass
    # what 32-bit byte offsets reach; the oracle checks 3 sampled heads.
    w = W["long-bf16"]
    cpu = problem(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.dtype,
                  w.seed, h0=True)
    got = run_gpu(cpu, w.chunk)
    heads = [0, 44, 79]
    hs = torch.tensor(heads)
    g_of = hs // (w.nheads // w.ngroups)
    sub = {"x": cpu["x"][:, :, hs], "dt": cpu["dt"][:, :, hs], "A": cpu["A"][hs],
           "B": cpu["B"][:, :, g_of], "C": cpu["C"][:, :, g_of], "D": cpu["D"][hs],
           "h0": cpu["h0"][:, hs], "dy": cpu["dy"][:, :, hs], "dfinal": cpu["dfinal"][:, hs]}
    ref = run_oracle(sub)
    got_s = {"dx": got["dx"][:, :, heads], "ddt": got["ddt"][:, :, heads],
             "dA": got["dA"][heads], "dD": got["dD"][heads], "dh0": got["dh0"][:, heads]}
    check("long-bf16 full size, heads " + str(heads), got_s, ref, "bf16",
          names=("dx", "ddt", "dA", "dD", "dh0"))


def test_backward_recompute_through_state_scan():
    # 4 x 64 heads of headdim 64 at whole 128-token chunks: 256 slices of 64 rows, where
    # the recomputed forward states come from the single-pass state kernel
    cpu = problem(4, 256, 64, 64, 128, 1, "bf16", seed=57)
    check("recompute via state scan", run_gpu(cpu, 256), run_oracle(cpu), "bf16")


# bf16 shapes of the matrix-core path beyond the workloads: headdim 128 (64-token chunks),
# one head per group (dB, dC written directly), heads per group with no head blocking (a
# reduce over every head) and with blocks of 2 heads summed in the kernel (then 4 blocks
# reduced)
@pytest.mark.parametrize("shape", [
    (1, 200, 4, 128, 64, 2, 64), (1, 150, 2, 128, 128, 1, 128), (2, 90, 4, 64, 64, 4, 256),
    (1, 300, 6, 64, 128, 2, 256), (2, 4096, 8, 64, 64, 1, 256)])
def test_backward_bf16_shapes(shape):
    b, L, H, P, S, G, T = shape
    cpu = problem(b, L, H, P, S, G, "bf16", seed=3 + L)
    check(f"bf16 shape {shape}", run_gpu(cpu, T), run_oracle(cpu), "bf16")


@pytest.mark.parametrize("dtype,T", [("bf16", 256), ("fp32", 64)])
def test_backward_extreme_decay(dtype, T):
    # dt up to 2 with A down to -16: per-token log2 decays near -46, so decays across a
    # 16-token tile leave the fp32 range; every factor the kernels form must stay <= 1
    g = torch.Generator()
    g.manual_seed(77)
    cpu = gen.draw(1, 300, 4, 64, 128, 2, gen.torch_dtype(dtype), g, random_h0=True,
                   dt_range=(0.05, 2.0), A_range=(1.0, 16.0))
    cpu.update(gen.draw_cotangents(1, 300, 4, 64, 128, g))
    got = run_gpu(cpu, T)
    for n in NAMES:
        assert torch.isfinite(got[n]).all(), n
    check(f"extreme decay {dtype}", got, run_oracle(cpu), dtype)


def test_backward_bf16_token_walks():
    # a bf16 shape with no matrix-core plan (headdim 32) takes the token walks
    cpu = problem(2, 300, 4, 32, 64, 2, "bf16", seed=41)
    check("bf16 walks (P=32)", run_gpu(cpu, 128), run_oracle(cpu), "bf16")


def test_backward_falls_back_within_size_limits():
    # 262144 tokens, 32 heads, dstate 256: 64-token chunk states would pass 2e9 elements,
    # so the backward runs the token walks at 256-token chunks; the oracle checks two
    # sampled heads (each its own group with the shared B, C)
    B_, L, H, P, S, G = 1, 262144, 32, 64, 256, 1
    cpu = problem(B_, L, H, P, S, G, "bf16", seed=9)
    got = run_gpu(cpu, 256)
    heads = [5, 30]
    hs = torch.tensor(heads)
    sub = {"x": cpu["x"][:, :, hs], "dt": cpu["dt"][:, :, hs], "A": cpu["A"][hs],
           "B": cpu["B"][:, :, [0, 0]], "C": cpu["C"][:, :, [0, 0]], "D": cpu["D"][hs],
           "h0": cpu["h0"][:, hs], "dy": cpu["dy"][:, :, hs], "dfinal": cpu["dfinal"][:, hs]}
    ref = run_oracle(sub)
    got_s = {"dx": got["dx"][:, :, heads], "ddt": got["ddt"][:, :, heads],
             "dA": got["dA"][heads], "dD": got["dD"][heads], "dh0": got["dh0"][:, heads]}
    check("size-limit fallback, heads " + str(heads), got_s, ref, "bf16",
          names=("dx", "ddt", "dA", "dD", "dh0"))
