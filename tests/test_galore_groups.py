"""GaLore parameter grouping (CPU): the rule of the Colossal-AI page's GaLore section
(2-D parameters projected with the group's rank fields; names with ``bias`` or
``LayerNorm.weight`` without weight decay; everything else plain AdamW)."""
import pytest
import torch

from memory_efficient_optimizers_amd import GaLoreAdamW, get_galore_param_groups


class Tiny(torch.nn.Module):
    def __init__(self):
        super().__init__()
        self.embed = torch.nn.Embedding(50, 16)
        self.proj = torch.nn.Linear(16, 32)
        self.LayerNorm = torch.nn.LayerNorm(32)
        self.conv = torch.nn.Conv1d(4, 4, 3)
        self.scale = torch.nn.Parameter(torch.ones(7))


def test_groups_follow_the_page_rule():
    m = Tiny()
    groups = get_galore_param_groups(m, weight_decay=1e-2, rank=8, update_proj_gap=50, scale=0.5)
    names = {id(p): n for n, p in m.named_parameters()}
    by = [sorted(names[id(p)] for p in g["params"]) for g in groups]
    assert by[0] == ["embed.weight", "proj.weight"]
    assert groups[0]["rank"] == 8 and groups[0]["update_proj_gap"] == 50 and groups[0]["scale"] == 0.5
    assert groups[0]["proj_type"] == "std" and groups[0]["weight_decay"] == 1e-2
    assert by[1] == ["conv.weight", "scale"] and "rank" not in groups[1] and groups[1]["weight_decay"] == 1e-2
    assert by[2] == ["LayerNorm.bias", "LayerNorm.weight", "conv.bias", "proj.bias"]
    assert groups[2]["weight_decay"] == 0.0 and "rank" not in groups[2]


def test_defaults_and_validation():
    m = Tiny()
    groups = get_galore_param_groups(m, weight_decay=0.0)
    assert groups[0]["rank"] == 256 and groups[0]["update_proj_gap"] == 200 and groups[0]["scale"] == 0.25
    opt = GaLoreAdamW(groups)
    assert opt.defaults["lr"] == 1e-3 and opt.defaults["betas"] == (0.9, 0.999) and opt.defaults["eps"] == 1e-8
    with pytest.raises(ValueError):
        GaLoreAdamW([dict(params=[torch.nn.Parameter(torch.zeros(3, 3))], rank=2, proj_type="reverse")])
    GaLoreAdamW([dict(params=[torch.nn.Parameter(torch.zeros(3, 3))], rank=2, proj_type="reverse_std")])
    with pytest.raises(ValueError):
        GaLoreAdamW(groups, lr=-1.0)
