"""The seeded input generators: determinism, recipe, and bf16 rounding."""
import json
import os

import numpy as np
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_lengths_match_fixture():
    with open(os.path.join(GOLDEN, "workload_lengths.json")) as f:
        fx = json.load(f)
    for s in range(5):
        assert workloads.lognormal_lengths(32768, s, 32768) == fx[f"longtail_seed{s}"]
    assert workloads.zigzag_pack_lengths(0) == fx["zigzag_pack_seed0"]


def test_longtail_seed0_shape():
    ls = workloads.lognormal_lengths(32768, 0, 32768)
    assert sum(ls) == 32768 and len(ls) == 30
    assert ls[:10] == [788, 521, 1794, 762, 273, 1149, 5188, 2931, 209, 85]
    assert min(ls) >= 1 and max(ls) == 5733


def test_lognormal_median_is_page_value():
    with open(os.path.join(GOLDEN, "page_examples.json")) as f:
        med = json.load(f)["corpus_median_length"]["median"]
    assert workloads.synth.MEDIAN_LEN == med
    # many untruncated draws: the empirical median sits near 644
    ls = workloads.lognormal_lengths(10_000_000, 123, 10_000_000)[:-1]
    assert abs(np.median(ls) / med - 1) < 0.05


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(100_000, dtype=np.float32) * rng.choice([1e-3, 1, 1e3], 100_000).astype(np.float32)
    # include exact ties: low 16 bits == 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_cu_seqlens():
    cu = workloads.cu_from_lengths([5, 17, 42])
    assert cu.dtype == np.int32 and cu.tolist() == [0, 5, 22, 64]


def test_tiny_pack_deterministic():
    a, b = workloads.tiny_pack(), workloads.tiny_pack()
    assert np.array_equal(a["q"], b["q"]) and a["q"].shape == (64, 2, 64)
    assert a["cu_seqlens"].tolist() == [0, 5, 22, 64]


def test_shared_question_layout():
    packs = workloads.shared_question_packs(n_packs=2, question=16, answers=3, answer_len=8, heads=4,
                                            kv_heads=2, d=8)
    assert len(packs) == 2
    assert packs[0]["cu_seqlens"].tolist() == [0, 16, 24, 32, 40]
    assert not np.array_equal(packs[0]["q"], packs[1]["q"])
