"""sscan_ssd_fwd_noalloc (the SSD prompt scan on the library's static device scratch)
against sscan_ssd_fwd with a caller's workspace, through the C ABI: the same kernels
and plan, so the results must be bit-identical. Two calls in a row, the second on a
smaller problem, for the MFMA chunk paths, bf16 and fp32 (with state hand-offs between
segments in the scratch), and for the token-loop path (slice carries in the scratch); where
two passes would not fit the scratch the call takes one; a problem that needs more scratch
than there is is refused before any launch."""
import numpy as np
import pytest
import torch

from state_space_model_sscan_amd import binding as bd
from state_space_model_sscan_amd import inputs as gen

from _gpu import dev, par, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bd.lib()


def _args(inp):
    a = inp.act
    return (dev(inp.x, a), dev(inp.dt_raw, a), par(inp.dt_bias), par(inp.A_log), dev(inp.B, a), dev(inp.C, a),
            par(inp.D), dev(inp.z, a), par(inp.h0))


def _both(inp, want_states=False):
    args = _args(inp)
    y1, h1, s1 = bd.sscan_ssd_fwd(*args, want_states=want_states)
    st = torch.empty_like(s1) if want_states else None
    y2, h2, s2 = bd.sscan_ssd_fwd_noalloc(*args, states=st)
    torch.cuda.synchronize()
    assert torch.isfinite(y1.float()).all() and torch.isfinite(h1).all()
    assert torch.equal(y1, y2), "y differs"
    assert torch.equal(h1, h2), "state_output differs"
    if want_states:
        assert torch.equal(s1, s2), "states differ"


@pytest.mark.parametrize("seg", [0, 2])
def test_noalloc_chunk_path_two_calls(seg):
    """bf16, head_dim 64, state_dim 128: the chunk kernel's queues (and, with segments of
    two chunks, the state hand-offs) in the static scratch."""
    try:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, seg)
        big = gen.make_ssd(2, 1000, 8, 64, 128, 2, act="bf16", seed=91, gate=True, h0=True)
        small = gen.make_ssd(1, 300, 4, 64, 128, 1, act="bf16", seed=92, gate=False, h0=False)
        for inp in (big, small):
            say("noalloc chunk path", inp.x.shape, "segment chunks", seg)
            _both(inp)
    finally:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 0)


@pytest.mark.parametrize("seg", [0, 2])
def test_noalloc_f32_chunk_path_two_calls(seg):
    """fp32, head_dim 64, state_dim 128: the fp32 chunk kernel's queues, C B^T tiles and
    (with segments of two chunks) state hand-offs in the static scratch."""
    try:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, seg)
        big = gen.make_ssd(2, 900, 6, 64, 128, 2, act="f32", seed=191, gate=True, h0=True)
        small = gen.make_ssd(1, 200, 2, 64, 128, 1, act="f32", seed=192, gate=False, h0=False)
        for inp in (big, small):
            say("noalloc f32 chunk path", inp.x.shape, "segment chunks", seg)
            _both(inp)
    finally:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 0)


def test_noalloc_token_loop_path_two_calls():
    """fp32 on the token loop (the knob sends head_dim 64 / state_dim 128 there), long
    enough to be cut into slices whose carries live in the scratch; the second call is
    smaller, and a third asks for per-token states."""
    big = gen.make_ssd(1, 3000, 2, 64, 128, act="f32", seed=93, gate=True, h0=True)
    small = gen.make_ssd(1, 700, 1, 32, 64, act="f32", seed=94, gate=True, h0=False)
    try:
        bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 1)
        for inp in (big, small):
            say("noalloc token loop", inp.x.shape)
            _both(inp)
    finally:
        bd.set_tuning(bd.TUNE_SSD_F32_TOKEN_LOOP, 0)
    _both(gen.make_ssd(1, 100, 2, 64, 128, act="bf16", seed=95, gate=True, h0=True), want_states=True)


def test_noalloc_takes_one_pass_where_two_would_not_fit():
    """8 chains of 1024 chunks: the plan takes two passes, whose first-pass states and
    C B^T tiles need more than the static scratch; the allocation-free call takes one
    pass instead (C B^T tiles only: 10.5 MB), bit-identical to the workspace call forced
    to one pass, and is not refused."""
    inp = gen.make_ssd(1, 65536, 8, 64, 128, act="bf16", seed=98, gate=True, h0=True)
    args = _args(inp)
    say("noalloc one-pass fallback", inp.x.shape)
    try:
        bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 1)
        y1, h1, _ = bd.sscan_ssd_fwd(*args)
    finally:
        bd.set_tuning(bd.TUNE_SSD_TWO_PASS, 0)
    y2, h2, _ = bd.sscan_ssd_fwd_noalloc(*args)
    torch.cuda.synchronize()
    assert torch.isfinite(y1.float()).all() and torch.isfinite(h1).all()
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


def test_noalloc_refuses_a_problem_larger_than_the_scratch():
    """800 chains cut into one-chunk segments need 26 MB of hand-off states: refused with
    SSCAN_ERR_UNSUPPORTED before any launch; the outputs stay untouched."""
    inp = gen.make_ssd(2, 128, 400, 64, 128, act="bf16", seed=96, gate=False, h0=False)
    args = _args(inp)
    y = torch.full_like(args[0], 3.0)
    try:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 1)
        need = bd.sscan_ssd_workspace_size(bd.ssd_desc(args[0], args[4]))
        assert need > (16 << 20)
        with pytest.raises(bd.SscanError) as e:
            bd.sscan_ssd_fwd_noalloc(*args, y=y)
        assert e.value.name == "SSCAN_ERR_UNSUPPORTED"
        torch.cuda.synchronize()
        assert bool((y == 3.0).all())
    finally:
        bd.set_tuning(bd.TUNE_SSD_SEGMENT_CHUNKS, 0)
    # the scratch is still good afterwards
    _both(gen.make_ssd(1, 200, 2, 64, 128, act="bf16", seed=97, gate=True, h0=True))
