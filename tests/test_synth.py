"""The seeded input generators: determinism, storage rounding, and the
planted verification logits (CPU only)."""
import numpy as np
import torch

import oracle
from speculative_decoding_05_amd import configs, synth


def test_bf16_storage_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    assert np.array_equal(synth.bf16_bits_to_f32(bits), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_streams_are_deterministic_and_chunk_invariant():
    a = synth.normal(9, 1, synth.SHARED, (6, 5, 4), 0.02, "bf16", chunks=1)
    b = synth.normal(9, 1, synth.SHARED, (6, 5, 4), 0.02, "bf16", chunks=3)
    assert np.array_equal(a, b)
    c = synth.per_sequence(9, 3, 3, (7,), 1.0, "f32")
    d = synth.per_sequence(9, 3, 2, (7,), 1.0, "f32")
    assert np.array_equal(c[:2], d)          # sequence b does not depend on B


def test_verification_logits_plant_low_entropy_rows():
    cfg = configs.CONFIGS["tiny_f32"]
    tree = oracle.build_tree(oracle.dense_paths(cfg.K, cfg.k), cfg.K, cfg.k)
    g = np.random.default_rng(1)
    B = 4
    idx = np.stack([np.stack([g.choice(cfg.V, cfg.k, replace=False) for _ in range(B)]) for _ in range(cfg.K)])
    root = g.integers(0, cfg.V, B)
    z = synth.verification_logits(cfg.cfg_id, cfg.V, tree["parent"], tree["depth"], tree["rank"],
                                  idx, root, configs.acc_float, cfg.k)
    z2 = synth.verification_logits(cfg.cfg_id, cfg.V, tree["parent"], tree["depth"], tree["rank"],
                                   idx, root, configs.acc_float, cfg.k)
    assert z.dtype == np.float32 and z.shape == (B, tree["T"], cfg.V)
    assert np.array_equal(z, z2)
    for b in range(B):
        for n in range(tree["T"]):
            _, H, _ = oracle.row_distribution(z[b, n].astype(np.float64), 1.0)
            assert H < 4.0                        # far below ln V = 6.9
