"""The seeded generators give identical bytes for identical keys, distinct
streams for distinct keys, and the distributions the workloads name."""
import numpy as np

import datagen


def test_same_key_same_bytes():
    a = datagen.normal_f32((1, 2, 3), (64, 128), 0.02)
    b = datagen.normal_f32((1, 2, 3), (64, 128), 0.02)
    assert a.tobytes() == b.tobytes()
    c = datagen.normal_f32((1, 2, 4), (64, 128), 0.02)
    assert a.tobytes() != c.tobytes()


def test_bf16_generator_is_rne_of_fp32():
    f = datagen.normal_f32((5, 5), (10000,))
    b = datagen.bf16_bits_from_f32(f)
    back = datagen.bf16_bits_to_f32(b)
    # within half a bf16 ulp
    ulp = np.abs(np.spacing(back.astype(np.float32))) * 2 ** 16
    assert np.all(np.abs(back - f) <= ulp / 2)


def test_distributions():
    w, x = datagen.C1()
    assert w.dtype == np.float32 and w.shape == (1024, 1024)
    assert abs(w.std() - 0.02) < 2e-4
    assert x.dtype == np.uint16 and x.shape == (1, 1024)
    d = datagen.f16_lognormal((3, 2), (100000,), 0.5)
    assert abs(np.log(d.astype(np.float64)).std() - 0.5) < 0.01
    s = datagen.pm1_f32((3, 0), (1000, 100))
    assert set(np.unique(s)) == {-1.0, 1.0} and abs(s.mean()) < 0.01
    H = datagen.haar_orthogonal((5, 0), 64)
    assert np.allclose(H @ H.T, np.eye(64), atol=1e-12)
    c5 = datagen.C5(M=8)
    assert c5["H"].dtype == np.float32 and c5["x"].shape == (8, 4096)
