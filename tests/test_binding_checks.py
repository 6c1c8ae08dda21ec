"""The Python binding's argument checks, on the CPU: wrong dtypes, shapes, short caches and host
tensors raise ValueError before any library call (no kernel runs here)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
tq = pytest.importorskip("vector_quantization_amd")

D = 128


def _codec(bits=2, m=D):
    rot = np.eye(D, dtype=np.float32)
    sk = np.ones((m, D), np.float32) if m else None
    c, t = tq.make_codebook(D, bits)
    return tq.codec_from_arrays(D, bits, m, rot, sk, c, t, device="cpu")


def _codes(codec, n):
    return tq.alloc_codes(codec, n, device="cpu")


def test_scores_checks():
    kc = _codec()
    codes = _codes(kc, 2 * 2 * 10)
    q = torch.zeros((2, 4, D))
    with pytest.raises(ValueError, match="float32"):
        tq.scores(kc, q.to(torch.bfloat16), codes, 10, 2)
    with pytest.raises(ValueError, match="records"):
        tq.scores(kc, q, _codes(kc, 39), 10, 2)
    with pytest.raises(ValueError, match="multiple"):
        tq.scores(kc, torch.zeros((2, 3, D)), codes, 10, 2)
    with pytest.raises(ValueError, match="shape"):
        tq.scores(kc, q, codes, 10, 2, logits=torch.zeros((2, 4, 9)))
    with pytest.raises(ValueError, match="contiguous"):
        tq.scores(kc, torch.zeros((4, 2, D)).transpose(0, 1), codes, 10, 2)
    with pytest.raises(ValueError, match="CUDA"):
        tq.scores(kc, q, codes, 10, 2)
    bad = tq.Codes(codes.idx, None, codes.norms)
    with pytest.raises(ValueError, match="sign"):
        tq.scores(kc, q, bad, 10, 2)
    narrow = tq.Codes(codes.idx[:, :16], codes.sign, codes.norms)
    with pytest.raises(ValueError, match="contiguous|bytes"):
        tq.scores(kc, q, narrow, 10, 2)


def test_attend_and_decode_step_checks():
    kc, vc = _codec(), _codec(3, 0)
    n_seq, hq, hkv, cap = 2, 8, 2, 16
    kcodes, vcodes = _codes(kc, n_seq * hkv * cap), _codes(vc, n_seq * hkv * cap)
    q = torch.zeros((n_seq, hq, D))
    with pytest.raises(ValueError, match="records"):
        tq.attend_decode(kc, vc, q, kcodes, _codes(vc, n_seq * hkv * cap - 1), cap, hkv, 0.1)
    with pytest.raises(ValueError, match="CUDA"):
        tq.attend_decode(kc, vc, q, kcodes, vcodes, cap, hkv, 0.1)
    kn = torch.zeros((n_seq, hkv, D), dtype=torch.bfloat16)
    pos = torch.zeros(n_seq, dtype=torch.int32)
    with pytest.raises(ValueError, match="int32"):
        tq.decode_step(kc, vc, q, kn, kn, pos.long(), cap, 1e4, kcodes, vcodes, 0.1)
    with pytest.raises(ValueError, match="shape"):
        tq.decode_step(kc, vc, q, kn, kn, pos[:1], cap, 1e4, kcodes, vcodes, 0.1)
    with pytest.raises(ValueError, match="dtype"):
        tq.decode_step(kc, vc, q, kn, kn.float(), pos, cap, 1e4, kcodes, vcodes, 0.1)
    with pytest.raises(ValueError, match="records"):
        tq.decode_step(kc, vc, q, kn, kn, pos, cap + 1, 1e4, kcodes, vcodes, 0.1)
    with pytest.raises(ValueError, match="CUDA"):
        tq.decode_step(kc, vc, q, kn, kn, pos, cap, 1e4, kcodes, vcodes, 0.1)
    with pytest.raises(ValueError, match="records"):
        tq.append(kc, kn, pos, cap + 1, 1e4, kcodes)
    with pytest.raises(ValueError, match="int32"):
        tq.append(kc, kn, pos.float(), cap, 1e4, kcodes)


def test_encode_and_search_checks():
    kc = _codec()
    x = torch.zeros((10, D))
    with pytest.raises(ValueError, match="float32, float16 or bfloat16"):
        tq.encode(kc, x.to(torch.int32))
    with pytest.raises(ValueError, match=r"\[\.\.\., 128\]"):
        tq.encode(kc, torch.zeros((10, 64)))
    with pytest.raises(ValueError, match="records"):
        tq.encode(kc, x, out=_codes(kc, 9))
    with pytest.raises(ValueError, match="float32"):
        tq.encode(kc, x.half(), pre_rotated=True)
    with pytest.raises(ValueError, match="CUDA"):
        tq.encode(kc, x)
    with pytest.raises(ValueError, match="records"):
        tq.search_topk(kc, torch.zeros((3, D)), _codes(kc, 99), 100, 10)
    with pytest.raises(ValueError, match="k must"):
        tq.search_topk(kc, torch.zeros((3, D)), _codes(kc, 100), 100, 33)


def test_polar_checks():
    tabs = np.zeros((7, 4, 4), np.float32)
    pc = tq.polar_codec_from_arrays(D, 2, np.eye(D, dtype=np.float32), tabs, device="cpu")
    codes = tq.alloc_polar_codes(pc, 40, device="cpu")
    q = torch.zeros((2, 4, D))
    with pytest.raises(ValueError, match="float32"):
        tq.polar_scores(pc, q.half(), codes, 10, 2)
    with pytest.raises(ValueError, match="records"):
        tq.polar_scores(pc, q, tq.alloc_polar_codes(pc, 39, device="cpu"), 10, 2)
    with pytest.raises(ValueError, match="CUDA"):
        tq.polar_scores(pc, q, codes, 10, 2)
    vc = _codec(3, 0)
    with pytest.raises(ValueError, match="records"):
        tq.polar_attend_decode(pc, vc, q, codes, _codes(vc, 39), 10, 2, 0.1)
