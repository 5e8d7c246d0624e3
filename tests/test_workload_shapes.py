"""Shape sanity of the synthetic workloads against the counts the pages print
(not parity: these check that the configurations are read the way the pages
size the models, and that the benchmark's FLOP count is twice the activated
parameters).

Sources: the cheat sheet "Mixture of Experts and Hybrid Architectures"
("DeepSeek-V3 config", "Models side by side", "Formulas") and "Lesson 2 --
From the Dense FFN to a Layer of Experts", section 3.
"""
import math

from synthetic import WORKLOADS

B = 1e9


def swiglu_params(d, F):
    return 3 * d * F  # W1, W3 [F][d] and W2 [d][F]


def test_deepseek_v3_expert_parameters_fit_the_printed_totals():
    # 61 layers = 3 dense + 58 MoE; 671B total, 37B active (cheat sheet)
    w = WORKLOADS["dsv3_prefill"]
    assert (w.d, w.E, w.k, w.F, w.Fs) == (7168, 256, 8, 2048, 2048)
    moe_layers = 58
    per_layer_routed = w.E * swiglu_params(w.d, w.F)
    assert per_layer_routed == 11_274_289_152
    total_experts = moe_layers * (per_layer_routed + swiglu_params(w.d, w.Fs))
    active_experts = moe_layers * (w.k + 1) * swiglu_params(w.d, w.F)
    assert total_experts < 671 * B and total_experts > 0.95 * 671 * B  # experts hold nearly all of it
    assert active_experts < 37 * B
    # sparsity of the whole model: 37/671, about 5.5 %
    assert abs(37 / 671 - 0.055) < 0.001


def test_decode_shape_shares_the_prefill_layer():
    a, b = WORKLOADS["dsv3_prefill"], WORKLOADS["dsv3_decode"]
    assert (a.d, a.E, a.k, a.F, a.Fs, a.score_fn, a.n_groups, a.topk_groups, a.route_scale) == \
        (b.d, b.E, b.k, b.F, b.Fs, b.score_fn, b.n_groups, b.topk_groups, b.route_scale)
    assert b.T == 64


def test_mixtral_expert_ratio_bounds_the_model_ratio():
    # 47B total / 13B active; experts alone scale as E / k, the rest (attention,
    # embeddings) is paid on every token, so the model's ratio sits below E / k
    w = WORKLOADS["mixtral_e8_top2"]
    assert (w.E, w.k, w.d, w.F) == (8, 2, 4096, 14336)
    assert 47 / 13 < w.E / w.k


def test_fine_grained_expert_sets():
    # C(256, 8), about 400 trillion selections per token
    n = math.comb(256, 8)
    assert n == 409_663_695_276_000
    assert abs(n / 400e12 - 1) < 0.03


def test_layer_flops_are_twice_the_activated_parameters():
    # one multiply-add per activated weight per token: router E*d, k routed
    # SwiGLUs and the shared one
    for w in WORKLOADS.values():
        active = w.E * w.d + w.k * swiglu_params(w.d, w.F) + (swiglu_params(w.d, w.Fs) if w.Fs else 0)
        assert w.flops == 2.0 * w.T * active, w.name
    w = WORKLOADS["dsv3_prefill"]
    assert abs(w.flops / w.T / 1e6 - 796.4) < 0.1  # MFLOP per token
