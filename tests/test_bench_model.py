"""The benchmark's byte model and scheduling choices, on the CPU (no GPU call).

`bench.py` prices every call by algorithmic bytes (each lookup's row counted once, every
input read and every output written once); these tests pin those figures to the per-call
values the workload definitions imply, worked out by hand below, so that the roofline's
`achieved` cannot drift from its definition.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from embedding_lookup_feature_amd import synth  # noqa: E402


def test_training_step_bytes_per_call():
    wl = synth.WORKLOADS["train_step"]  # B 65536, 26 fp32 tables x 128, bf16 activations
    B, F, D, S = 65536, 26, 128, 480
    assert (wl.batch, wl.num_tables, wl.dim, wl.out_stride) == (B, F, D, S)
    nnz = B * F  # one lookup per bag
    a = bench.algorithmic_bytes(wl, nnz)
    # rows (fp32) + indices + offsets + pooled output (bf16)
    assert a["emb_bag_fwd"] == 1_703_936 * 512 + 4 * 1_703_936 + 4 * (1_703_937) + B * F * D * 2
    assert round(a["emb_bag_fwd"] / 1e9, 3) == 1.322
    # x0 + pooled vectors in, interaction rows out
    assert a["dot_interact_fwd"] == B * 27 * D * 2 + B * S * 2
    assert round(a["dot_interact_fwd"] / 1e6, 1) == 515.9
    # gradient rows in, x0 + pooled vectors in, their gradients out
    assert a["dot_interact_bwd"] == B * S * 2 + 2 * B * 27 * D * 2
    assert round(a["dot_interact_bwd"] / 1e6, 1) == 968.9
    # the fused forward storing the pooled vectors: the gather's bytes plus x0 in and the
    # interaction rows out (the pooled vectors are not read back from HBM)
    assert a["emb_dot_fwd"] == a["emb_bag_fwd"] + B * D * 2 + B * S * 2
    # the backward rebuilding them: rows, indices and offsets in place of the pooled vectors
    assert a["emb_dot_bwd"] == B * S * 2 + B * D * 2 + 1_703_936 * 512 + 8 * 1_703_936 + 4 + B * 27 * D * 2
    assert round(a["emb_dot_bwd"] / 1e9, 3) == 1.419


def test_forward_only_stores_no_pooled_vectors():
    wl = synth.WORKLOADS["fwd_core"]
    nnz = wl.batch * wl.num_tables
    a = bench.algorithmic_bytes(wl, nnz)
    assert a["emb_dot_fwd"] == a["emb_bag_fwd"] - wl.batch * wl.num_tables * wl.dim * 2 \
        + wl.batch * wl.dim * 2 + wl.batch * wl.out_stride * 2
    assert round(a["emb_dot_fwd"] / 1e9, 3) == 0.966


def test_sort_start_policy():
    # one lookup per bag: 3 x 8-bit passes over 1.7M pairs (82 MB) hide behind the 969 MB
    # interaction backward; multi-hot: 4 passes over 32.8M pairs (2.1 GB) do not
    tr = synth.WORKLOADS["train_step"]
    mh = synth.WORKLOADS["multi_hot"]
    assert bench.sort_start(tr, tr.batch * tr.num_tables) == "bwd"
    assert bench.sort_start(mh, 32_770_000) == "fwd"


def test_fused_backward_coverage():
    assert bench.fused_bwd_ok(synth.WORKLOADS["train_step"])
    assert not bench.fused_bwd_ok(synth.WORKLOADS["multi_hot"])  # 101 vectors
    assert not bench.fused_bwd_ok(synth.WORKLOADS["tiny"])       # fp32, D = 16


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_roofline_names_the_kernel_the_shape_runs():
    assert bench.kernel_of("dot_interact_bwd", synth.WORKLOADS["train_step"]) == "k_dot_bwd_mfma"
    assert bench.kernel_of("dot_interact_bwd", synth.WORKLOADS["multi_hot"]) == "k_dot_bwd_mfma"
    assert bench.kernel_of("dot_interact_bwd", synth.WORKLOADS["tiny"]) == "k_dot_bwd_valu"       # fp32
    assert bench.kernel_of("dot_interact_bwd", synth.WORKLOADS["train_small_tables"]) == "k_dot_bwd_valu"  # D = 16
    assert bench.kernel_of("dot_interact_fwd", synth.WORKLOADS["tiny"]) == "k_dot_fwd_valu"
    assert bench.kernel_of("dot_interact_fwd", synth.WORKLOADS["train_small_tables"]) == "k_dot_fwd_mfma"
    assert bench.kernel_of("dot_interact_fwd", synth.WORKLOADS["multi_hot"]) == "k_dot_fwd_wide"  # 101 vectors


def test_every_path_kernel_has_its_sources_listed():
    """The counter summary's validity check hashes each kernel's sources: every kernel of the
    gather, interaction, sort and update files must be in that map."""
    import re
    csrc = os.path.join(ROOT, "embedding_lookup_feature_amd", "csrc")
    for f in ("emb_bag_fwd.hip", "dot_interact.hip", "emb_dot_fwd.hip", "grad_sort.hip", "grad_update.hip"):
        text = open(os.path.join(csrc, f)).read()
        names = set(re.findall(r"\bvoid\s+(k_[a-z0-9_]+)\s*\(", text))  # kernels are void k_*
        assert names, f
        for k in names:
            if k.startswith(("k_scan_", "k_seg_flags", "k_seg_emit", "k_seg_empty")):
                continue  # the segment listing of emb_grad_sort: not on the timed path
            assert k in bench.KERNEL_SOURCES, (f, k)
            assert f"embedding_lookup_feature_amd/csrc/{f}" in bench.KERNEL_SOURCES[k], (f, k)


def test_source_digest_ignores_comments_only():
    a = bench.source_digest(["embedding_lookup_feature_amd/csrc/grad_update.hip"])
    path = os.path.join(ROOT, "embedding_lookup_feature_amd", "csrc", "grad_update.hip")
    text = open(path).read()
    import hashlib
    import re
    stripped = re.sub(r"//[^\n]*", " ", re.sub(r"/\*.*?\*/", " ", text, flags=re.S))
    assert a == hashlib.sha256(" ".join(stripped.split()).encode()).hexdigest()
    assert a != hashlib.sha256(" ".join((stripped + " x").split()).encode()).hexdigest()


def test_long_bag_gather_is_named():
    assert bench.kernel_of("emb_bag_fwd", synth.WORKLOADS["multi_hot"]) == "k_emb_bag_long"
    assert bench.kernel_of("emb_bag_fwd", synth.WORKLOADS["train_step"]) == "k_emb_bag_fwd"
