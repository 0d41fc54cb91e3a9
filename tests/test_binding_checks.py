"""The Python binding checks every buffer before a pointer reaches the C ABI,
which carries no sizes: a buffer that is too small, of the wrong dtype, on
another device or not contiguous raises ValueError and nothing is called.
Tensors live on the meta device here (no memory, no GPU); every case below
fails before the library would be reached."""
import pytest
import torch

import softmax_matrix_cores_amd as fs

B, H, S, D = 1, 2, 100, 128
DEV = torch.device("meta")


def mx(elem, rows, axis, shrink_codes=0, shrink_scales=0, dtype=torch.uint8, device=DEV, prescale=1.0):
    cb, sb = fs.mx_sizes(elem, B * H, rows, D, axis)
    return fs.MXTensor(torch.empty(cb - shrink_codes, dtype=dtype, device=device),
                       torch.empty(sb - shrink_scales, dtype=torch.uint8, device=device), fs._elem(elem), prescale)


def operands(**kw):
    q = kw.pop("q", None) or mx("e2m3", S, 0, prescale=fs.fold_prescale(D ** -0.5))
    k = kw.pop("k", None) or mx("e2m3", S, 0)
    v = kw.pop("v", None) or mx("e2m3", S, 1)
    return q, k, v


def call(q, k, v, **kw):
    return fs.forward(q, k, v, B, H, S, S, D, D ** -0.5, "e2m3", **kw)


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_short_codes_or_scales(which):
    axis = 1 if which == "v" else 0
    with pytest.raises(ValueError, match="codes"):
        call(*operands(**{which: mx("e2m3", S, axis, shrink_codes=1)}))
    with pytest.raises(ValueError, match="scales"):
        call(*operands(**{which: mx("e2m3", S, axis, shrink_scales=1)}))


def test_operand_dtype_device_and_layout():
    with pytest.raises(ValueError, match="uint8"):
        call(*operands(k=mx("e2m3", S, 0, dtype=torch.int8)))
    with pytest.raises(ValueError, match="must be on"):
        call(*operands(v=mx("e2m3", S, 1, device=torch.device("cpu"))))
    q, k, v = operands()
    cb = q.codes.numel()
    q.codes = torch.empty(2 * cb, dtype=torch.uint8, device=DEV)[::2]
    with pytest.raises(ValueError, match="contiguous"):
        call(q, k, v)
    # an operand is sized by the format it declares: FP4-sized codes declared FP8
    bad = mx("e2m1", S, 0)
    bad.elem = fs.ELEMS["e4m3"]
    with pytest.raises(ValueError, match="codes"):
        call(*operands(k=bad))


def test_output_and_counts():
    q, k, v = operands()
    with pytest.raises(ValueError, match="out"):
        call(q, k, v, out=torch.empty(B, H, S, D, dtype=torch.float16, device=DEV))
    with pytest.raises(ValueError, match="out"):
        call(q, k, v, out=torch.empty(B, H, S - 1, D, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError, match="counts"):
        call(q, k, v, counts=torch.empty(B * H * S - 1, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError, match="counts"):
        call(q, k, v, counts=torch.empty(B * H * S, dtype=torch.int64, device=DEV))


def test_p_dump_window_and_buffers():
    q, k, v = operands()
    s32 = (S + 31) // 32 * 32
    ok_c = torch.empty(8 * s32, dtype=torch.uint8, device=DEV)
    ok_s = torch.empty(8 * s32 // 32, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError, match="window"):
        call(q, k, v, p_dump=(0, H, 0, 8, ok_c, ok_s))
    with pytest.raises(ValueError, match="window"):
        call(q, k, v, p_dump=(0, 0, 8, 8, ok_c, ok_s))
    with pytest.raises(ValueError, match="p_dump codes"):
        call(q, k, v, p_dump=(0, 0, 0, 9, ok_c, ok_s))
    with pytest.raises(ValueError, match="p_dump scales"):
        call(q, k, v, p_dump=(0, 0, 0, 8, ok_c, ok_s[:-1]))


def test_shape_arguments():
    q, k, v = operands()
    with pytest.raises(ValueError, match="shape"):
        fs.forward(q, k, v, B, H, S, S, 96, D ** -0.5, "e2m3")
    with pytest.raises(ValueError, match="shape"):
        fs.forward(q, k, v, B, H, S, 0, D, D ** -0.5, "e2m3")
    # operands sized for fewer heads than the call names
    with pytest.raises(ValueError):
        fs.forward(q, k, v, B, H + 1, S, S, D, D ** -0.5, "e2m3")


def test_bf16_baseline_inputs():
    q = torch.empty(B, H, S, D, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="k and v"):
        fs.forward_bf16_baseline(q, torch.empty(B, H, S, 64, dtype=torch.bfloat16, device=DEV), q, D ** -0.5)
    with pytest.raises(ValueError, match="bfloat16"):
        fs.forward_bf16_baseline(q, q.float(), q, D ** -0.5)
    kt = torch.empty(B, H, D, S, dtype=torch.bfloat16, device=DEV).transpose(2, 3)  # [B,H,S,D], strided
    with pytest.raises(ValueError, match="contiguous"):
        fs.forward_bf16_baseline(q, kt, q, D ** -0.5)
    with pytest.raises(ValueError, match="out"):
        fs.forward_bf16_baseline(q, q, q, D ** -0.5, out=torch.empty(B, H, S, D, dtype=torch.float32, device=DEV))
