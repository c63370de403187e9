"""The bound the tile-maxima top-k relies on, checked on the CPU.

Tile images are dealt to 1024 threads in order (tile t to thread t mod 1024),
and the 64 sets {lane l of every 64-lane wave} each take their largest image.
theta is the largest set maximum that at least k set maxima reach.  Then the
row's k largest values (ties broken by the smaller index) must all lie in
tiles whose image reaches theta, and have an image of at least theta.  This
checks that claim by brute force over random rows, tied rows and short rows;
it exercises no GPU code."""
import numpy as np
import pytest

NT = 1024


def images(x):
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u[u == 0x80000000] = 0
    return np.where((u & 0x80000000) != 0, ~u, u | np.uint32(0x80000000)).astype(np.uint64)


def theta_of(tile_img, k):
    nt = len(tile_img)
    per_set = np.zeros(64, dtype=np.uint64)
    for t in range(nt):
        s = (t % NT) % 64
        per_set[s] = max(per_set[s], tile_img[t])
    reach = [(per_set >= g).sum() for g in per_set]
    ok = [g for g, r in zip(per_set, reach) if r >= k]
    return max(ok) if ok else 0


@pytest.mark.parametrize("V,k,kind", [(32000, 10, "normal"), (32000, 64, "normal"), (5003, 17, "ties"),
                                      (1000, 2, "normal"), (70001, 64, "ties"), (33, 4, "normal"),
                                      (17, 5, "ties"), (5, 5, "normal"), (1, 1, "normal"), (2048, 33, "zeros")])
def test_top_k_lies_in_tiles_reaching_theta(V, k, kind):
    g = np.random.default_rng(V * 131 + k)
    for _ in range(5):
        x = g.standard_normal(V).astype(np.float32)
        if kind == "ties":
            x = (np.round(x * 2) / 2).astype(np.float32)
        elif kind == "zeros":
            x[:] = 0.0
            x[::3] = -0.0
        im = images(x)
        nt = (V + 15) // 16
        padded = np.zeros(nt * 16, dtype=np.uint64)
        padded[:V] = im
        tile_img = padded.reshape(nt, 16).max(axis=1)
        theta = theta_of(tile_img, k)
        # the k largest by (image desc, index asc)
        top = sorted(range(V), key=lambda i: (-int(im[i]), i))[:k]
        for i in top:
            assert im[i] >= theta
            assert tile_img[i // 16] >= theta
        # and at least k elements of the candidate tiles reach theta
        cand = [i for i in range(V) if tile_img[i // 16] >= theta and im[i] >= theta]
        assert len(cand) >= k
