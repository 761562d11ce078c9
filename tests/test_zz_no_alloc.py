"""The no-allocation fit (dbscan_fit_device_noalloc, fixed per-GPU scratch)
against the workspace fit (dbscan_fit_device) through the C ABI: labels and
counts bit-identical, on two calls in a row, the second with a smaller
input (the scratch keeps the first call's contents), then a third call as
large as the scratch allows and one past it."""
import numpy as np
import pytest

from all_pairs_distance_amd import datagen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible gfx950 device"
    import all_pairs_distance_amd as apd
    return torch, apd


def _pair(torch, apd, x, eps, m):
    """(labels, counts) from the workspace entry and from the no-allocation
    entry on the same device points and stream."""
    n, d = x.shape
    xt = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    stream = torch.cuda.current_stream()
    out = []
    ws = apd.Workspace(n, d, max_edges=n * 64)
    lab = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    st = apd.dbscan_fit_device(xt.data_ptr(), n, d, eps, m, lab.data_ptr(),
                               cnt.data_ptr(), ws.ptr, ws.nbytes,
                               stream.cuda_stream)
    assert st == 0, st
    out.append((lab.cpu().numpy(), cnt.cpu().numpy()))
    lab2 = torch.full((n,), -9, dtype=torch.int32, device="cuda")
    cnt2 = torch.full((n,), -9, dtype=torch.int32, device="cuda")
    st = apd.dbscan_fit_device_noalloc(xt.data_ptr(), n, d, eps, m,
                                       lab2.data_ptr(), cnt2.data_ptr(),
                                       stream.cuda_stream)
    assert st == 0, st
    out.append((lab2.cpu().numpy(), cnt2.cpu().numpy()))
    return out


def test_noalloc_matches_workspace_fit_twice_then_smaller(env, orc):
    torch, apd = env
    x1, eps1, m1, _ = datagen.make_workload(2)           # 50,000 x 2
    x2 = datagen.gaussian_blobs(3000, 3, seed=8, n_blobs=4, sigma=0.02,
                                noise_frac=0.2)           # smaller, other d
    for name, x, eps, m in (("first", x1, eps1, m1),
                            ("second_smaller", x2, 0.03, 5)):
        print(f"noalloc case {name} n={x.shape[0]} d={x.shape[1]}", flush=True)
        (la, ca), (lb, cb) = _pair(torch, apd, x, eps, m)
        assert np.array_equal(ca, cb), f"{name}: counts differ"
        assert np.array_equal(la, lb), f"{name}: labels differ"
        if x.shape[0] <= 3000:
            want_l, want_c, _ = orc.fit(x, eps, m)
            assert np.array_equal(cb, want_c) and np.array_equal(lb, want_l)


def test_noalloc_at_the_size_limit(env):
    torch, apd = env
    d = 8
    n = 1000
    while apd.dbscan_workspace_bytes(2 * n, d) <= apd.NOALLOC_SCRATCH_BYTES:
        n *= 2
    x = datagen.gaussian_blobs(n, d, seed=31, n_blobs=10, sigma=0.03,
                               noise_frac=0.1)
    print(f"noalloc limit case n={n} d={d}", flush=True)
    (la, ca), (lb, cb) = _pair(torch, apd, x, 0.05, 6)
    assert np.array_equal(ca, cb) and np.array_equal(la, lb)
    big = n
    while apd.dbscan_workspace_bytes(big, d) <= apd.NOALLOC_SCRATCH_BYTES:
        big *= 2
    xt = torch.zeros((big, d), dtype=torch.float32, device="cuda")
    lab = torch.empty(big, dtype=torch.int32, device="cuda")
    st = apd.dbscan_fit_device_noalloc(xt.data_ptr(), big, d, 0.05, 6,
                                       lab.data_ptr(), None,
                                       torch.cuda.current_stream().cuda_stream)
    assert st == apd.ERR_TOO_LARGE
