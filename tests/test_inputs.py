"""The seeded input generator: determinism, exact counts, and bf16 round-to-nearest-even."""
import numpy as np
import torch

from workloads import (WORKLOADS, draw_labels, f32_to_bf16_bits, make_ce_inputs,
                       make_flce_inputs, random_ce)


def test_rne_matches_torch_cast():
    x = np.random.default_rng(0).normal(0, 3, 100000).astype(np.float32)
    # exact ties: low half 0x8000 with both parities of the kept bit
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], dtype=np.uint32).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_same_seed_same_bytes_and_seed_matters():
    a = random_ce(700, 333, seed=5)
    b = random_ce(700, 333, seed=5)
    c = random_ce(700, 333, seed=6)
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.labels, b.labels)
    assert not np.array_equal(a.logits, c.logits)


def test_exact_ignored_counts_and_label_range():
    for name, w in WORKLOADS.items():
        d = draw_labels(w, 0)
        assert d.labels.dtype == np.int32 and d.labels.shape == (w.n,)
        ignored = int((d.labels == -100).sum())
        expect = int(round(w.ignore_frac * w.n))
        if w.documents:
            assert d.doc_starts.size == w.documents and d.doc_starts[0] == 0
            assert np.all(np.diff(d.doc_starts) > 0)
            assert np.all(d.labels[d.doc_starts] == -100)
            assert ignored == w.documents
        else:
            assert ignored == expect, name
        ok = d.labels[d.labels != -100]
        assert ok.min() >= 0 and ok.max() < w.v


def test_small_workloads_shapes_and_spike():
    w = WORKLOADS["ce_64x1000"]
    inp = make_ce_inputs(w)
    assert inp.logits.shape == (64, 1000) and inp.logits.dtype == np.uint16
    assert int((inp.labels == -100).sum()) == 6
    w3 = WORKLOADS["flce_2048x768x32777"]
    f = make_flce_inputs(w3)
    assert f.hidden.shape == (2048, 768) and f.weight.shape == (32777, 768)
    assert f.bias.dtype == np.float32 and f.bias.shape == (32777,)
    assert int((f.labels == -100).sum()) == 41


def test_spike_lands_on_label_column():
    from workloads import Workload
    w = Workload("spiky", 77, "ce", n=600, v=50, chunk_size=64, logit_sigma=0.5,
                 spike=8.0, spike_frac=0.3, ignore_frac=0.05)
    inp = make_ce_inputs(w)
    vals = (inp.logits.astype(np.uint32) << 16).view(np.float32)
    d = inp.draw
    assert d.spike_rows.size == 180
    assert np.all(vals[d.spike_rows, d.spike_cols] > 5.0)
