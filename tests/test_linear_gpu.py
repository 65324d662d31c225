"""Int4Linear and int4_linear on MI355X against the CPU oracle.

One layer: y = act(x @ w_hat.T + b) within the matmul bound (fp32 output)
plus the binary16 rounding of the output (fp16 output). A stack of layers
(the engine page's two-layer model, and MLP blocks of the c3 and c4 shapes)
against the oracle applied layer by layer with the same fp16 rounding of each
hidden activation; the allowed error of the second layer carries the first
layer's bound through the second layer's weights. Every expected value and
every bound is computed from oracle outputs only.
"""
import os

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3
H_ULP = 2.0 ** -11          # relative spacing bound of binary16 (normal range)
H_SUB = 2.0 ** -25          # half the smallest binary16 subnormal


@pytest.fixture(scope="module")
def L():
    from dequantizing_gemm_amd import linear
    return linear


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy() if t.dtype == torch.float16 else t.cpu().numpy()


def say(*a):
    print(*a, flush=True)


def oracle_layer(x, w, b, group, affine, relu):
    """Oracle quantization of w and the oracle layer output: (y, pre-activation
    bound, w_hat as float64, codes)."""
    if affine:
        p, s, z, K = oracle.quantize_int4_affine(w, group)
    else:
        (p, s, K), z = oracle.quantize_int4(w, group), None
    y, bound = oracle.int4_matmul_ex(x.astype(np.float32), p, s, K, group, bias=b, relu=relu,
                                     with_bound=True, zeros=z)
    wh = oracle.dequantize_int4(p, s, K, group, np.float32, zeros=z).astype(np.float64)
    return y.astype(np.float64), bound, wh, (p, s, z)


def allowed(y_ref, bound, has_bias, half_out):
    """Bound on |y_gpu - y_ref| for one layer given exact inputs."""
    e = TOL * bound + (2.0 ** -22 * np.abs(y_ref) if has_bias else 0.0)
    if half_out:
        e = e + H_ULP * (np.abs(y_ref) + e) + H_SUB
    return e


def weights(N, K, seed, scale=0.05):
    return (np.random.default_rng(seed).normal(size=(N, K)) * scale).astype(np.float32)


@pytest.mark.parametrize("affine", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.float16])
def test_layer_matches_oracle(L, affine, out_dtype):
    say(f"case: Int4Linear 1024->384 g128 affine={affine} out={out_dtype}")
    N, K, g = 384, 1024, 128
    w = weights(N, K, 1)
    b = np.random.default_rng(2).normal(size=N).astype(np.float32)
    layer = L.Int4Linear.from_float(dev(w), dev(b), group=g, affine=affine, relu=True, out_dtype=out_dtype)
    _, _, _, (p, s, z) = oracle_layer(np.zeros((1, K), np.float16), w, b, g, affine, True)
    assert np.array_equal(host(layer.packed), p)
    assert np.array_equal(layer.scales.cpu().numpy().view(np.uint16), s.view(np.uint16))
    if affine:
        assert np.array_equal(host(layer.zeros), z)
    for M in (1, 3, 5, 16, 40, 300):
        x = np.random.default_rng(M).normal(size=(M, K)).astype(np.float16)
        y = layer(dev(x))
        assert y.dtype == out_dtype and tuple(y.shape) == (M, N)
        y_ref, bound, _, _ = oracle_layer(x, w, b, g, affine, True)
        err = np.abs(host(y).astype(np.float64) - y_ref)
        assert np.all(err <= allowed(y_ref, bound, True, out_dtype == torch.float16)), M
    # leading dimensions are flattened and restored
    x3 = np.random.default_rng(9).normal(size=(2, 3, K)).astype(np.float16)
    y3 = host(layer(dev(x3)))
    y2 = host(layer(dev(x3.reshape(6, K))))
    assert y3.shape == (2, 3, N) and np.array_equal(y3.reshape(6, N), y2)


def test_layer_fp32_x_fp16_out(L):
    """fp32 activations (the generic kernel) with fp16 output, odd K and a
    ragged last group."""
    say("case: Int4Linear fp32 x, fp16 out, K=301 g=5")
    N, K, g = 40, 301, 5
    w = weights(N, K, 11)
    for affine in (False, True):
        layer = L.Int4Linear.from_float(dev(w), group=g, affine=affine, out_dtype=torch.float16)
        x = np.random.default_rng(12).normal(size=(3, K)).astype(np.float32)
        y_ref, bound, _, _ = oracle_layer(x, w, None, g, affine, False)
        err = np.abs(host(layer(dev(x))).astype(np.float64) - y_ref)
        assert np.all(err <= allowed(y_ref, bound, False, True)), affine


def test_dequantized_weight(L):
    say("case: Int4Linear.dequantized_weight")
    w = weights(96, 200, 3)
    for affine in (False, True):
        layer = L.Int4Linear.from_float(dev(w), group=32, affine=affine)
        _, _, wh, _ = oracle_layer(np.zeros((1, 200), np.float16), w, None, 32, affine, False)
        assert np.array_equal(host(layer.dequantized_weight()).astype(np.float64), wh)


def chain_check(layers_cfg, x, L, seed=0, edit=None):
    """Build the stack on the GPU and on the oracle side; check each layer's
    output with the error carried from the layer before. edit(w, g), if
    given, changes each layer's float weights in place before quantization."""
    rng = np.random.default_rng(seed)
    mods, ws = [], []
    for (K, N, g, affine, relu, out16) in layers_cfg:
        w = weights(N, K, int(rng.integers(1 << 30)), scale=1.0 / np.sqrt(K))
        if edit is not None:
            edit(w, g)
        b = (rng.normal(size=N) * 0.1).astype(np.float32)
        mods.append(L.Int4Linear.from_float(dev(w), dev(b), group=g, affine=affine, relu=relu,
                                            out_dtype=torch.float16 if out16 else torch.float32))
        ws.append((w, b))
    model = torch.nn.Sequential(*mods)
    y_gpu = host(model(dev(x))).astype(np.float64)

    h_ref = x.astype(np.float64)          # oracle input of the current layer
    d_in = np.zeros_like(h_ref)           # bound on |GPU input - oracle input|
    for (K, N, g, affine, relu, out16), (w, b) in zip(layers_cfg, ws):
        y_ref, bound, wh, _ = oracle_layer(h_ref.astype(np.float32), w, b, g, affine, relu)
        carried = d_in @ np.abs(wh).T                       # from the input difference
        own = TOL * (bound + carried) + 2.0 ** -22 * (np.abs(y_ref) + carried)
        e = own + carried                                   # GPU output vs y_ref, before rounding
        if out16:
            h_next = y_ref.astype(np.float16).astype(np.float64)   # the oracle's own fp16 rounding
            e = e + H_ULP * (np.abs(y_ref) + e) + H_SUB + np.abs(h_next - y_ref)
            y_ref = h_next
        h_ref, d_in = y_ref, e
    err = np.abs(y_gpu - h_ref)
    worst = float(np.max(err / np.maximum(d_in, 1e-300)))
    assert np.all(err <= d_in), f"worst ratio {worst:.3e}"
    return worst


def test_engine_two_layer_model(L):
    """The engine page's example: 256 -> 128 -> 10 with ReLU on both layers,
    x [4, 256], block 128 (here fp16 activations and an fp16 hidden layer)."""
    say("case: two-layer model 256->128->10")
    x = np.random.default_rng(42).normal(size=(4, 256)).astype(np.float16)
    for affine in (True, False):
        chain_check([(256, 128, 128, affine, True, True), (128, 10, 128, affine, True, False)], x, L)


@pytest.mark.parametrize("M", [1, 16, 300])
def test_c3_mlp_stack(L, M):
    """c3's MLP block (768 -> 3072 -> 768, groups 64 and 32) as a stack of two
    layers, ReLU after the first, fp16 between them."""
    say(f"case: c3 MLP stack M={M}")
    x = np.random.default_rng(M).normal(size=(M, 768)).astype(np.float16)
    chain_check([(768, 3072, 64, False, True, True), (3072, 768, 32, False, False, False)], x, L, seed=M)


@pytest.mark.parametrize("M", [1, 16])
def test_c4_mlp_stack(L, M):
    """c4's MLP shapes (4096 -> 11008 -> 4096, group 128): decode-sized
    inputs through the gemv and skinny kernels."""
    say(f"case: c4 MLP stack M={M}")
    x = np.random.default_rng(100 + M).normal(size=(M, 4096)).astype(np.float16)
    chain_check([(4096, 11008, 128, False, True, True), (11008, 4096, 128, True, False, False)], x, L,
                seed=M)


def edge_rows(w, g):
    """The method's edge cases in a layer's weights: zero first, middle and
    last groups, a row of -8 * 2^-24 (binary16 scale 0x0001, every code -8),
    and a row a thousand times larger than the rest (scales near 4)."""
    G = w.shape[1] // g
    w[0, :g] = 0.0
    w[1, (G // 2) * g:(G // 2 + 1) * g] = 0.0
    w[2, (G - 1) * g:] = 0.0
    w[3, :] = -8.0 * 2.0 ** -24
    w[4, :] *= 1000.0


@pytest.mark.parametrize("M", [1, 16, 300])
def test_stack_edge_rows(L, M):
    """A stack of two layers whose weights hold the edge rows, through the
    gemv (M = 1), skinny (M = 16) and tiled (M = 300) kernels, symmetric then
    affine codes, fp16 between the layers."""
    say(f"case: stack with edge rows M={M}")
    x = np.random.default_rng(500 + M).normal(size=(M, 512)).astype(np.float16)
    chain_check([(512, 384, 128, False, True, True), (384, 256, 64, True, False, False)], x, L, seed=M,
                edit=edge_rows)


def test_persistence_round_trip(L, tmp_path):
    say("case: save_int4 / load_int4 on the GPU")
    model = torch.nn.Sequential(
        L.Int4Linear.from_float(dev(weights(512, 256, 5)), dev(np.ones(512, np.float32)), group=64,
                                relu=True, out_dtype=torch.float16),
        L.Int4Linear.from_float(dev(weights(64, 512, 6)), None, group=128, affine=True))
    p = os.path.join(tmp_path, "stack.safetensors")
    L.save_int4(p, model)
    fresh = torch.nn.Sequential(
        L.Int4Linear(256, 512, group=64, relu=True, out_dtype=torch.float16, device=DEV),
        L.Int4Linear(512, 64, group=128, bias=False, affine=True, device=DEV))
    L.load_int4(p, fresh)
    x = dev(np.random.default_rng(7).normal(size=(8, 256)).astype(np.float16))
    assert np.array_equal(host(model(x)).view(np.uint32), host(fresh(x)).view(np.uint32))
    loaded = L.load_int4(p, device=DEV)
    y = loaded["1"](loaded["0"](x))
    assert np.array_equal(host(model(x)).view(np.uint32), host(y).view(np.uint32))
