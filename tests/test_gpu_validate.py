"""The debug idx check (sla_validate_idx, and SLA_VALIDATE=1 in front of the entry points that
read idx): well-formed lists pass, and each kind of malformed list is refused before anything
reads it.  Out-of-range entries go only to sla_validate_idx itself, never to a forward."""

import os

import pytest
import torch

import block_sparse_linear_02_amd as sla
import gen
from tests import cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def case():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sla.lib()
    wl = gen.workload("video_l", H=2, N=1800, grid=(1, 45, 40), topk=5).with_(name="validate", wid=7)
    c = cases.make_case(wl, gap=False)
    d = torch.device("cuda:0")
    g = {n: c[n].to(d) for n in ("Q", "K", "V", "alpha", "Wq", "Wk")}
    idx, _, _ = sla.route(g["Q"], g["K"], g["Wq"], g["Wk"], 5)
    torch.cuda.synchronize()
    return g, idx


@pytest.fixture
def validate_env():
    old = os.environ.get("SLA_VALIDATE")
    os.environ["SLA_VALIDATE"] = "1"
    yield
    if old is None:
        del os.environ["SLA_VALIDATE"]
    else:
        os.environ["SLA_VALIDATE"] = old


def test_router_output_is_well_formed(case):
    g, idx = case
    assert sla.validate_idx(g["Q"], idx)
    assert sla.validate_idx(g["Q"], idx[..., :0].contiguous())  # topk = 0


@pytest.mark.parametrize("kind", ["past_end", "negative", "duplicate", "descending"])
def test_malformed_lists_are_refused(case, kind):
    g, idx = case
    nb = idx.shape[2]
    bad = idx.clone()
    if kind == "past_end":
        bad[0, 1, nb - 1, -1] = nb
    elif kind == "negative":
        bad[0, 0, 3, 0] = -1
    elif kind == "duplicate":
        bad[0, 1, 7, 2] = bad[0, 1, 7, 1]
    else:
        bad[0, 0, 0, 0], bad[0, 0, 0, 1] = idx[0, 0, 0, 1], idx[0, 0, 0, 0]
    assert not sla.validate_idx(g["Q"], bad)
    assert sla.validate_idx(g["Q"], idx)  # the word holds nothing over from the bad call


def test_validate_env_guards_forward_and_backward(case, validate_env):
    g, idx = case
    ref = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode="mask_product")
    torch.cuda.synchronize()
    bad = idx.clone()
    bad[0, 1, 4, 0], bad[0, 1, 4, 1] = idx[0, 1, 4, 1], idx[0, 1, 4, 0]  # in range, not ascending
    for mode in ("fused", "mask_product"):
        with pytest.raises(sla.SLAError) as e:
            sla.forward(g["Q"], g["K"], g["V"], bad, g["alpha"], linear_mode=mode)
        assert e.value.status == sla.SLA_ERR_INVALID
    dO = torch.ones_like(g["Q"])
    with pytest.raises(sla.SLAError) as e:
        sla.backward(g["Q"], g["K"], g["V"], bad, g["alpha"], dO)
    assert e.value.status == sla.SLA_ERR_INVALID
    again = sla.forward(g["Q"], g["K"], g["V"], idx, g["alpha"], linear_mode="mask_product")
    torch.cuda.synchronize()
    assert torch.equal(again, ref)
