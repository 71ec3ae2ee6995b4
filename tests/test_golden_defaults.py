"""The workloads take over the parameters the page prints (tests/golden/page_defaults.json,
page "DLRM For PyTorch", section Command-line options)."""
import inspect
import json
import os

import bench
from embedding_lookup_feature_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_defaults.json")))


def val(key):
    return GOLD[key]["value"]


def test_headline_workloads_use_the_synthetic_dataset_tables_and_embedding_dim():
    for name in ("fwd_core", "train_step", "fwd_core_uniform", "fwd_core_distinct"):
        wl = synth.WORKLOADS[name]
        assert list(wl.rows) == val("synthetic_dataset_table_sizes"), name
        assert wl.dim == val("embedding_dim"), name


def test_mlp_sizes_and_numerical_features():
    wl = synth.WORKLOADS["train_step"]
    assert wl.bottom_mlp[0] == val("num_numerical_features")
    assert list(wl.bottom_mlp[1:]) == val("bottom_mlp_sizes")
    assert list(synth.TOP_MLP) == val("top_mlp_sizes")


def test_generator_base_seed_is_the_page_seed():
    assert synth.BASE_SEED == val("seed")


def test_inference_sweep_covers_the_page_batch_sizes():
    sizes = inspect.signature(bench.inference_sweep).parameters["sizes"].default
    assert set(val("inference_benchmark_batch_sizes")) <= set(sizes)


def test_interaction_ops_built():
    # dot (and its fused forms) and cat are built; cuda_dot names the page's own CUDA kernel
    # of the dot interaction, which the dot calls stand in for
    from embedding_lookup_feature_amd import embcore as ec
    names = set(ec.header_functions())
    assert {"dot_interact_fwd", "dot_interact_bwd", "cat_interact_fwd", "cat_interact_bwd"} <= names
    assert {"dot", "cat"} <= set(val("interaction_ops"))
