"""The seeded input generator: determinism, quantiser correctness, layouts."""
import math

import numpy as np
import torch

import synth


def test_normal_is_counter_based_and_standard():
    a = synth.normal(5, 200000)
    b = synth.normal(5, 1000, offset=5000)
    assert (a[5000:6000] == b).all()
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    assert not (synth.normal(6, 1000) == a[:1000]).all()


def test_thread_count_does_not_change_output():
    A1, s1 = synth.act(3, 100, 512, threads=1)
    A8, s8 = synth.act(3, 100, 512, threads=7)
    assert (A1 == A8).all() and (s1 == s8).all()
    B1, t1 = synth.weight(4, 300, 256, threads=1)
    B8, t8 = synth.weight(4, 300, 256, threads=5)
    assert (B1 == B8).all() and (t1 == t8).all()


def test_encoder_roundtrips_every_finite_code():
    vals = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float()
    for c in range(256):
        v = float(vals[c])
        if math.isnan(v):
            continue
        assert synth.e4m3_encode(v) == c or (v == 0 and synth.e4m3_encode(v) in (0, 0x80))


def test_encoder_matches_torch_rne_in_range():
    x = np.concatenate([synth.normal(9, 20000) * 100, synth.normal(10, 5000) * 0.01]).astype(np.float32)
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([synth.e4m3_encode(float(v)) for v in x], np.uint8)
    assert (got == ref).all()


def test_scales_are_block_amax_over_448():
    M, K = 20, 384
    A, sa = synth.act(12, M, K)
    x = synth.normal(12, M * K).reshape(M, K)
    amax = np.abs(x.reshape(M, K // 128, 128)).max(axis=2)  # [M, Kb]
    assert np.array_equal(sa, (amax / np.float32(448)).T.astype(np.float32))
    # the largest element of every block lands on +-448
    assert (np.abs(A.reshape(M, K // 128, 128) & 0x7F).max(axis=2) == 0x7E).all()
    N = 200
    B, sb = synth.weight(13, N, K)
    y = synth.normal(13, N * K).reshape(N, K)
    for nb in range(2):
        for kb in range(3):
            blk = y[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert sb[nb, kb] == np.float32(np.abs(blk).max()) / np.float32(448)


def test_heavy_rows_and_layouts():
    rm = synth.heavy_rows(1, 4096)
    assert (rm == 50).sum() == 41 and (rm == 1).sum() == 4096 - 41
    A, sa = synth.act(2, 256, 256, row_mult=rm[:256])
    A0, sa0 = synth.act(2, 256, 256)
    heavy = rm[:256] == 50
    assert (A[heavy] == A0[heavy]).all()  # scaling a block does not change its codes
    assert np.allclose(sa[:, heavy], sa0[:, heavy] * 50, rtol=1e-6)
    idx, segs = synth.contiguous_indices(5, 8, 32768, uniform=False)
    assert idx.shape == (32768,) and sum(s[1] for s in segs) == 32768
    for g, (start, plen, valid) in enumerate(segs):
        assert start % 128 == 0 and plen % 128 == 0 and plen >= 128 and plen - valid < 128
        assert (idx[start:start + valid] == g).all() and (idx[start + valid:start + plen] == -1).all()
    idx4, _ = synth.contiguous_indices(5, 4, 32768, uniform=True)
    assert (np.bincount(idx4) == 8192).all()
    mm = synth.masked_counts(7, 16, 256)
    assert mm.min() >= 0 and mm.max() <= 256 and len(set(mm.tolist())) > 4
