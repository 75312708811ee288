"""GPU parity of the SVD codec initialisation (lla_svd_init) against the fp64
oracle (numpy SVD of the centred calibration rows).

What is unique is compared as such: the mean, the singular values, the
leading singular vectors where the spectrum separates them (sign fixed by
the same convention on both sides), and the codec's reconstruction error on
the calibration rows (optimal by Eckart-Young).  Where singular values
cluster, individual vectors are not unique: there the subspace's captured
energy is compared.  The loop slices must equal W_down's rows bit for bit."""
import sys

import numpy as np
import pytest
import torch

import looped_transformer_decode_amd as L
from oracle import lla_oracle as O
from synth import gen
from tests.gpu_cases import from_device, to_device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def spectrum_rows(seed, n, K, sv, offset=1.0):
    """Rows with prescribed singular values sv (after centring, roughly) plus
    a constant offset: Z diag(sv) V^T with orthonormal V."""
    rng = np.random.default_rng(seed)
    V, _ = np.linalg.qr(rng.standard_normal((K, len(sv))))
    Z = rng.standard_normal((n, len(sv))) / np.sqrt(n)
    return Z * np.asarray(sv)[None, :] @ V.T + offset * rng.standard_normal(K)[None, :]


def run_init(x_exact, dtype, G, T, width, r, device, iters=0):
    """x_exact: [n, G, K] float64 values exact in dtype."""
    n, _, K = x_exact.shape
    x = to_device(x_exact, dtype, device)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    mu = torch.empty((G, K), dtype=torch.float32, device=device)
    wd = torch.empty((G, K, r), dtype=tdt, device=device)
    wu = torch.empty((T, G, width, r), dtype=tdt, device=device)
    sig = torch.empty((G, r), dtype=torch.float32, device=device)
    L.lla_svd_init(x, T, width, r, mu, wd, wu, sig, iters=iters)
    torch.cuda.synchronize()
    return (mu.cpu().numpy().astype(np.float64), from_device(wd), from_device(wu),
            sig.cpu().numpy().astype(np.float64))


def check_codec(xg, T, width, r, mu, wd, wu, sig, dtype, sep=None, tol_sig=1e-4, tol_vec=2e-3):
    """One codec g: xg [n, K] exact rows; GPU outputs for it."""
    K = T * width
    omu, oW, oUp, osig = O.svd_init(xg, T, width, r)
    assert np.abs(mu - omu).max() <= 1e-5 * (np.abs(omu).max() + 1e-3)
    # loop slices are W_down's rows, bit for bit
    for t in range(T):
        assert np.array_equal(wu[t], wd[t * width:(t + 1) * width])
    # orthonormal columns (to the rounding of the stored type)
    gram = wd.T @ wd
    assert np.abs(gram - np.eye(r)).max() <= (1e-4 if dtype == "f32" else 2.5e-2)
    # singular values, relative to the largest
    s_err = np.abs(sig - osig).max() / osig[0]
    # leading vectors where the spectrum separates them
    nsep = r if sep is None else sep
    v_err = np.abs(wd[:, :nsep] - oW[:, :nsep]).max()
    # Eckart-Young: the codec's error on its calibration rows
    e_gpu = O.codec_error(xg, mu, wd, [wd[t * width:(t + 1) * width] for t in range(T)])
    e_opt = O.codec_error(xg, omu, oW, oUp)
    say(f"    sigma err {s_err:.2e}  vec err {v_err:.2e}  codec error {e_gpu:.6e} "
        f"(optimum {e_opt:.6e})")
    assert s_err <= tol_sig
    assert v_err <= tol_vec
    # bf16 W_down perturbs the projector by its rounding (about 1e-3 relative
    # per entry): at most ~1e-5 of the centred energy; 1e-4 allowed.
    assert e_gpu <= e_opt * (1 + 1e-3) + (1e-4 if dtype == "bf16" else 1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_separated_spectrum(device, dtype):
    """Per-head shapes, three codecs, well-separated singular values: every
    vector is unique up to sign."""
    G, T, width, r, n = 3, 4, 8, 6, 300
    K = T * width
    sv = 40.0 * 0.7 ** np.arange(K)
    x = np.stack([spectrum_rows(100 + g, n, K, sv) for g in range(G)], axis=1)
    x = gen.as_storage(x, dtype)[1]
    say(f"[svd] separated {dtype} G={G} K={K} r={r} n={n}")
    mu, wd, wu, sig = run_init(x, dtype, G, T, width, r, device)
    for g in range(G):
        check_codec(x[:, g], T, width, r, mu[g], wd[g], wu[:, g], sig[g], dtype,
                    tol_vec=2e-3 if dtype == "f32" else 8e-3)


def test_trajectory_rank8(device):
    """Long-recurrence codec shapes (T = 16, d = 128, r = 48, bf16): rank-8
    loop trajectories plus N(0, 0.05^2) noise.  The 8 signal directions are
    compared as vectors; the 40 noise directions by captured energy."""
    G, T, width, r, n = 2, 16, 128, 48, 4096
    K = T * width
    x = np.stack([gen.low_rank_trajectory(4, 5000 + g, n, K) for g in range(G)], axis=1)
    x = gen.as_storage(x, "bf16")[1]
    say(f"[svd] trajectory bf16 G={G} K={K} r={r} n={n}")
    mu, wd, wu, sig = run_init(x, "bf16", G, T, width, r, device)
    for g in range(G):
        check_codec(x[:, g], T, width, r, mu[g], wd[g], wu[:, g], sig[g], "bf16", sep=8,
                    tol_sig=5e-3, tol_vec=1e-2)


def test_lla2d_stack(device):
    """One LLA-2D codec: the stack is [t][h][d] of width H*d."""
    G, T, width, r, n = 1, 4, 128, 64, 1024
    K = T * width
    sv = np.concatenate([60.0 * 0.8 ** np.arange(16), np.full(K - 16, 0.5)])
    x = spectrum_rows(7, n, K, sv)[:, None, :]
    x = gen.as_storage(x, "bf16")[1]
    say(f"[svd] lla2d bf16 K={K} r={r} n={n}")
    mu, wd, wu, sig = run_init(x, "bf16", G, T, width, r, device)
    check_codec(x[:, 0], T, width, r, mu[0], wd[0], wu[:, 0], sig[0], "bf16", sep=16,
                tol_sig=5e-3, tol_vec=1e-2)


@pytest.mark.parametrize("n,K,r", [(10, 32, 12), (200, 16, 16), (64, 24, 1), (80, 12, 5)],
                         ids=["rank_deficient", "full_rank", "rank_one", "k_not_multiple_of_8"])
def test_edge_cases(device, n, K, r):
    """Fewer rows than the rank (centred rank n - 1 < r), r = K, r = 1, and a
    stack length that is not a multiple of 8 (the Gram matrix then comes from
    the generic tiled product with the centring in its loader)."""
    T, width = 2, K // 2
    rng = np.random.default_rng(n + K)
    x = gen.as_storage(rng.standard_normal((n, 1, K)) * 2 + 1, "f32")[1]
    say(f"[svd] edge n={n} K={K} r={r}")
    mu, wd, wu, sig = run_init(x, "f32", 1, T, width, r, device)
    omu, oW, oUp, osig = O.svd_init(x[:, 0], T, width, r)
    assert np.abs(mu[0] - omu).max() < 1e-5
    assert np.abs(wd[0].T @ wd[0] - np.eye(r)).max() < 1e-3
    e_gpu = O.codec_error(x[:, 0], mu[0], wd[0], [wd[0][t * width:(t + 1) * width] for t in range(T)])
    e_opt = O.codec_error(x[:, 0], omu, oW, oUp)
    say(f"    codec error {e_gpu:.3e} (optimum {e_opt:.3e})")
    assert e_gpu <= e_opt + 1e-5
    k = min(r, n - 1)
    assert np.abs(sig[0][:k] - osig[:k]).max() <= 1e-4 * osig[0]


def test_bf16_stack_not_multiple_of_8(device):
    """bf16 rows whose stack length (K = 12) is not a whole number of 16-byte
    vectors: the column means and the Gram matrix then take their
    element-wise forms."""
    T, width, r, n = 2, 6, 5, 120
    K = T * width
    rng = np.random.default_rng(12)
    x = gen.as_storage(rng.standard_normal((n, 1, K)) * 2 + 1, "bf16")[1]
    say(f"[svd] bf16 K={K} r={r} n={n}")
    mu, wd, wu, sig = run_init(x, "bf16", 1, T, width, r, device)
    omu, oW, oUp, osig = O.svd_init(x[:, 0], T, width, r)
    assert np.abs(mu[0] - omu).max() <= 1e-5 * (np.abs(omu).max() + 1e-3)
    assert np.abs(wd[0].T @ wd[0] - np.eye(r)).max() < 2e-2  # bf16 W_down
    assert np.abs(sig[0] - osig).max() <= 1e-4 * osig[0]
    e_gpu = O.codec_error(x[:, 0], mu[0], wd[0], [wd[0][t * width:(t + 1) * width] for t in range(T)])
    e_opt = O.codec_error(x[:, 0], omu, oW, oUp)
    say(f"    codec error {e_gpu:.4e} (optimum {e_opt:.4e})")
    assert e_gpu <= e_opt * (1 + 2e-2) + 1e-6  # W_down rounded to bf16


@pytest.mark.parametrize("r", [101, 79], ids=["block_117_odd", "block_95_odd"])
def test_large_odd_block(device, r):
    """Iterated blocks of odd order beyond what the small cases reach:
    m = r + 16 = 117 (the eigenvector matrix no longer fits LDS beside the
    Rayleigh-Ritz matrix, 8 x 8 registers per thread in the Cholesky step)
    and m = 95 (6 x 6).  The leading r singular values are distinct but close
    and the rest well below, so only the subspace is unique: compared are mu,
    sigma, orthonormality and the codec error against the optimum."""
    G, T, width, n = 2, 2, 80, 600
    K = T * width
    sv = np.concatenate([np.linspace(50.0, 20.0, r), np.full(K - r, 0.5)])
    x = np.stack([spectrum_rows(900 + g + r, n, K, sv) for g in range(G)], axis=1)
    x = gen.as_storage(x, "f32")[1]
    say(f"[svd] large odd block G={G} K={K} r={r} m={r + 16} n={n}")
    mu, wd, wu, sig = run_init(x, "f32", G, T, width, r, device)
    for g in range(G):
        omu, oW, oUp, osig = O.svd_init(x[:, g], T, width, r)
        assert np.abs(mu[g] - omu).max() <= 1e-5 * (np.abs(omu).max() + 1e-3)
        assert np.abs(wd[g].T @ wd[g] - np.eye(r)).max() < 1e-3
        for t in range(T):
            assert np.array_equal(wu[t, g], wd[g][t * width:(t + 1) * width])
        assert np.abs(sig[g] - osig).max() <= 1e-4 * osig[0]
        e_gpu = O.codec_error(x[:, g], mu[g], wd[g],
                              [wd[g][t * width:(t + 1) * width] for t in range(T)])
        e_opt = O.codec_error(x[:, g], omu, oW, oUp)
        say(f"    codec {g}: error {e_gpu:.4e} (optimum {e_opt:.4e})")
        assert e_gpu <= e_opt * (1 + 1e-4) + 1e-7


def test_deterministic(device):
    G, T, width, r, n = 2, 4, 16, 8, 256
    K = T * width
    x = gen.as_storage(np.random.default_rng(3).standard_normal((n, G, K)), "bf16")[1]
    a = run_init(x, "bf16", G, T, width, r, device)
    b = run_init(x, "bf16", G, T, width, r, device)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
