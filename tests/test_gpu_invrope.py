"""GPU parity of the inverse RoPE (csa_inverse_rope) against the oracle.

Tolerance, from the arithmetic: each rotated value is x c + y s (or y c - x s)
in FP32 with one fused multiply-add, so before rounding it is within
2^-23 (|x c| + |y s|) of the exact value, and BF16 rounding to nearest even
adds at most half an ulp, 2^-8 of the result (8 significant bits); copied
channels are bit-exact.
"""
import numpy as np
import pytest

import oracle
import synthetic
from tests import harness as H
from tests.tiny import bf16_bits

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _csa():
    import compressed_sparse_attention_csa_amd as csa
    csa.load()
    return csa


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _check(g, x, c, s, off, nt, what):
    """g: GPU BF16 values (float64); x: input BF16 values (float64)."""
    o = oracle.inverse_rope(x, c, s, off, nt)
    half = c.shape[1]
    tol = np.zeros_like(o)
    if half:
        span = slice(off, off + 2 * half)
        xs = x[:nt, :, span]
        mag = np.abs(xs[..., 0::2]) + np.abs(xs[..., 1::2])      # |x| + |y| per pair
        pair = np.repeat(mag, 2, axis=-1)
        tol[:nt, :, span] = 2.0 ** -8 * np.abs(o[:nt, :, span]) + 2.0 ** -22 * pair
    d = np.abs(g[:nt] - o[:nt])
    assert np.all(d <= tol[:nt]), f"{what}: worst {np.max(d - tol[:nt]):.3g} over"


@pytest.mark.parametrize("H_,D,R,off", [(8, 64, 16, 48), (5, 128, 64, 62), (64, 512, 64, 448),
                                        (3, 32, 0, 32), (16, 256, 256, 0)])
def test_inverse_rope_shapes(H_, D, R, off):
    print(f"[invrope] H={H_} D={D} R={R} off={off}", flush=True)
    csa = _csa()
    rng = np.random.default_rng(D + R + off)
    T, nt = 7, 5
    x_bits = bf16_bits(rng.standard_normal((T, H_, D)) * 3)
    ang = rng.uniform(-3, 3, (T, R // 2))
    c = np.cos(ang).astype(np.float32)
    s = np.sin(ang).astype(np.float32)
    c[1] = 1.0   # an identity row (rope position -1)
    s[1] = 0.0
    inp = _bf16(x_bits)
    out = torch.full_like(inp, 7.0)
    csa.csa_inverse_rope(inp, out, torch.as_tensor(c).cuda(), torch.as_tensor(s).cuda(), off, nt)
    torch.cuda.synchronize()
    x = H.bf16_to_f64(inp)
    g = H.bf16_to_f64(out)
    _check(g, x, c, s, off, nt, f"H{H_} D{D}")
    keep = np.ones(D, bool)
    keep[off:off + R] = False
    assert np.array_equal(out.view(torch.int16).cpu().numpy()[:nt][:, :, keep],
                          x_bits.view(np.int16)[:nt][:, :, keep])
    assert np.array_equal(out.view(torch.int16).cpu().numpy()[1], x_bits.view(np.int16)[1])
    assert torch.all(out[nt:] == 7.0)
    # in place gives the same bits
    inp2 = inp.clone()
    csa.csa_inverse_rope(inp2, inp2, torch.as_tensor(c).cuda(), torch.as_tensor(s).cuda(), off,
                         nt)
    torch.cuda.synchronize()
    assert torch.equal(inp2[:nt].view(torch.int16), out[:nt].view(torch.int16))
    assert torch.equal(inp2[nt:].view(torch.int16), inp[nt:].view(torch.int16))


def test_inverse_rope_after_the_c5_step():
    """The C5 step's attention output, rotated back with the step's own rope
    rows (rows at rope position -1 included in C3 and not in C5: both run)."""
    csa = _csa()
    for name in ("c5", "c3"):
        cfg = synthetic.get(name)
        print(f"[invrope] {cfg.name} step", flush=True)
        x = synthetic.make_inputs(cfg, seed=2).t
        step = csa.step_for_config(cfg, x)
        step.run()
        step.inv_rope()
        torch.cuda.synchronize()
        assert int(step.err.item()) == 0
        c = step.rope_cos.cpu().numpy()
        s = step.rope_sin.cpu().numpy()
        _check(H.bf16_to_f64(step.out_inv), H.bf16_to_f64(step.out), c, s, cfg.rope_offset,
               cfg.T, cfg.name)
