"""The text projection on the library's fixed device scratch
(sfm_text_project_noalloc, for callers that cannot allocate) against the
workspace form sfm_text_project: bitwise equal on two calls in a row, the
second with fewer tokens, and a shape beyond the scratch refused before any
launch."""

import sys

import pytest
import torch

from stream_flow_matching_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(*a):
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def sfm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from stream_flow_matching_amd import sfm as S
    S.lib()
    return S


def test_text_project_noalloc_equals_workspace_form(sfm):
    ctx = sfm.Context("ideogram4")
    k = synth.TEXT_FEATURES
    norm_w, wq, ws = synth.text_proj_params(4608, k, ("noalloc",))
    keep = (wq.to(DEV), ws.to(DEV), norm_w.to(DEV))
    w = sfm.qweight(sfm.SFM_W_FP8_E4M3, keep[0], keep[1])
    for M in (512, 77):                       # the second call is smaller
        _say("text project noalloc", M)
        raw = synth.text_raw(M, k, ("noalloc", M)).to(DEV)
        a = torch.empty(M, 4608, dtype=torch.bfloat16, device=DEV)
        b = torch.full((M, 4608), float("nan"), dtype=torch.bfloat16, device=DEV)
        sfm.sfm_text_project(ctx, raw, keep[2], w, a)
        sfm.sfm_text_project_noalloc(ctx, raw, keep[2], w, b)
        torch.cuda.synchronize()
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # 2048 tokens of 65,536 features need more than the 128 MiB scratch: refused on the host
    raw = torch.empty(1, dtype=torch.float32, device=DEV)
    big = torch.empty(2048, 65536, dtype=torch.float32, device=DEV)
    wbig_q = torch.empty(4608, 65536, dtype=torch.uint8, device=DEV)
    wbig = sfm.qweight(sfm.SFM_W_FP8_E4M3, wbig_q, keep[1])
    nw = torch.empty(65536, dtype=torch.bfloat16, device=DEV)
    out = torch.empty(2048, 4608, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sfm.SfmError) as e:
        sfm.sfm_text_project_noalloc(ctx, big, nw, wbig, out)
    assert "scratch" in str(e.value)
    del raw
