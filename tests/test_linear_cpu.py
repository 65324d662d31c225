"""Int4Linear host logic without a GPU: buffers, configuration, persistence
(round trip, checksums, configuration checks), and that the forward refuses
CPU tensors instead of computing anything on the CPU."""
import os

import pytest
import torch


def _mods():
    import __graft_entry__
    __graft_entry__._ensure_built()
    from dequantizing_gemm_amd import linear
    return linear


def _stack(L, seed=0):
    g = torch.Generator().manual_seed(seed)
    m = torch.nn.Sequential(
        L.Int4Linear(256, 128, group=64, relu=True, out_dtype=torch.float16, device="cpu"),
        L.Int4Linear(128, 10, affine=True, device="cpu"),
        L.Int4Linear(10, 3, group=4, bias=False, device="cpu"))
    for layer in m:
        layer.packed.copy_(torch.randint(0, 256, layer.packed.shape, generator=g, dtype=torch.uint8))
        layer.scales.copy_(torch.rand(layer.scales.shape, generator=g).half())
        if layer.zeros is not None:
            layer.zeros.copy_(torch.randint(0, 16, layer.zeros.shape, generator=g, dtype=torch.uint8))
        if layer.bias is not None:
            layer.bias.copy_(torch.randn(layer.bias.shape, generator=g))
    return m


def test_buffers_and_config():
    L = _mods()
    layer = L.Int4Linear(301, 48, group=128, affine=True, relu=True, out_dtype=torch.float16, device="cpu")
    assert tuple(layer.packed.shape) == (48, 151) and layer.packed.dtype == torch.uint8
    assert tuple(layer.scales.shape) == (48, 3) and layer.scales.dtype == torch.float16
    assert tuple(layer.zeros.shape) == (48, 3) and layer.zeros.dtype == torch.uint8
    assert tuple(layer.bias.shape) == (48,) and layer.bias.dtype == torch.float32
    assert layer.config() == {"in_features": 301, "out_features": 48, "group": 128, "bias": True,
                              "affine": True, "relu": True, "out_dtype": "float16"}
    plain = L.Int4Linear(64, 8, bias=False, device="cpu")
    assert plain.zeros is None and plain.bias is None
    assert set(plain.state_dict()) == {"packed", "scales"}
    with pytest.raises(ValueError):
        L.Int4Linear(64, 8, out_dtype=torch.bfloat16, device="cpu")
    with pytest.raises(ValueError):
        L.Int4Linear(0, 8, device="cpu")


def test_forward_refuses_cpu_tensors():
    L = _mods()
    layer = L.Int4Linear(64, 8, device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        layer(torch.zeros(2, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="features"):
        layer(torch.zeros(2, 63, dtype=torch.float16))


def test_save_load_round_trip(tmp_path):
    L = _mods()
    m = _stack(L)
    p = os.path.join(tmp_path, "m.safetensors")
    L.save_int4(p, m)
    m2 = _stack(L, seed=1)
    L.load_int4(p, m2, device="cpu")
    for (k, a), (k2, b) in zip(m.state_dict().items(), m2.state_dict().items()):
        assert k == k2 and torch.equal(a, b), k
    layers = L.load_int4(p, device="cpu")
    assert sorted(layers) == ["0", "1", "2"]
    assert layers["1"].config() == m[1].config()
    assert torch.equal(layers["1"].zeros, m[1].zeros) and layers["2"].bias is None
    # a single layer saves under the name "layer"
    L.save_int4(p, m[1])
    assert list(L.load_int4(p, device="cpu")) == ["layer"]


def test_load_detects_corruption_and_mismatch(tmp_path):
    L = _mods()
    m = _stack(L)
    p = os.path.join(tmp_path, "m.safetensors")
    L.save_int4(p, m)
    with pytest.raises(ValueError, match="configuration"):
        bad = _stack(L)
        bad[0] = L.Int4Linear(256, 128, group=64, relu=False, out_dtype=torch.float16, device="cpu")
        L.load_int4(p, bad, device="cpu")
    with pytest.raises(ValueError, match="no layer"):
        L.load_int4(p, torch.nn.Sequential(*list(_stack(L)), L.Int4Linear(3, 3, device="cpu")), device="cpu")
    raw = bytearray(open(p, "rb").read())
    raw[-1] ^= 0x01                                   # a byte of the last tensor's data
    q = os.path.join(tmp_path, "bad.safetensors")
    open(q, "wb").write(bytes(raw))
    with pytest.raises(ValueError, match="checksum"):
        L.load_int4(q, _stack(L), device="cpu")
    from safetensors.torch import save_file
    save_file({"a": torch.zeros(2)}, q, metadata={"format": "other"})
    with pytest.raises(ValueError, match="not an"):
        L.load_int4(q, device="cpu")
