"""MoeLayer's argument checks for expert-parallel shares, on the CPU (no
launch: the layer only records its arguments until forward)."""
import pytest
import torch

from mixture_experts_ffn_04_amd import binding as B


def _weights(E=16, E_loc=4, d=64, f=64):
    bf = torch.bfloat16
    return B.MoeWeights(torch.zeros(E, d, dtype=bf), None, torch.zeros(E_loc, 2 * f, d, dtype=bf),
                        torch.zeros(E_loc, d, f, dtype=bf))


def test_expert_ids_map():
    layer = B.MoeLayer(_weights(), 2, "softmax", expert_ids=[9, 2, 15, 4])
    m = layer.emap.tolist()
    assert m[9] == 0 and m[2] == 1 and m[15] == 2 and m[4] == 3
    assert sum(v == -1 for v in m) == 12


@pytest.mark.parametrize("kw", [
    dict(expert_ids=[1, 2, 3]),                 # fewer experts than the weights hold
    dict(expert_ids=[1, 2, 3, 3]),              # an expert twice
    dict(expert_ids=[1, 2, 3, 16]),             # past the router's experts
    dict(expert_ids=[-1, 2, 3, 4]),
    dict(expert_ids=[0, 1, 2, 3], experts=(0, 4)),
    dict(experts=(0, 5)),
    dict(experts=(13, 4)),                      # runs past expert 15
    dict(experts=(1, 4, 5)),                    # 1, 6, 11, 16: past expert 15
    dict(),                                     # a share's weights without a placement
    dict(experts=(0, 4), shared_part=(2, 2)),
])
def test_share_arguments_refused(kw):
    with pytest.raises(ValueError):
        B.MoeLayer(_weights(), 2, "softmax", **kw)


def test_strided_share_accepted():
    layer = B.MoeLayer(_weights(), 2, "softmax", experts=(3, 4, 4))      # 3, 7, 11, 15
    assert (layer.e_begin, layer.e_stride, layer.emap) == (3, 4, None)
