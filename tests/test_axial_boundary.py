"""The axial-block C entry points without a GPU: argument validation only
(axial_pass_validate makes no HIP call), and the Python wrapper's checks."""
import pytest
import torch

ROW, COL = 0, 1
OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3

# Stand-in addresses, never dereferenced, far apart so that nothing overlaps.
SZ = 1 << 34
X, OUT, LNW, LNB, WQKV, WOUT, BOUT = ((i + 1) * SZ for i in range(7))


def v(lib, x=X, out=OUT, ln_w=LNW, ln_b=LNB, w_qkv=WQKV, w_out=WOUT, b_out=BOUT, B=4, Hh=32,
      W=32, C=64, heads=4, axis=ROW, eps=1e-5):
    return lib.axial_pass_validate(x, out, ln_w, ln_b, w_qkv, w_out, b_out, B, Hh, W, C, heads,
                                   axis, eps)


def test_valid(hip_lib):
    assert v(hip_lib) == OK
    assert v(hip_lib, axis=COL) == OK
    assert v(hip_lib, out=X) == OK                    # in place
    assert v(hip_lib, W=1, Hh=64, axis=COL) == OK     # lengths 1 .. 64
    assert v(hip_lib, W=45, Hh=7) == OK
    assert v(hip_lib, eps=0.0) == OK


def test_invalid(hip_lib):
    for kw in (dict(x=0), dict(out=0), dict(ln_w=0), dict(ln_b=0), dict(w_qkv=0),
               dict(w_out=0), dict(b_out=0), dict(B=-1), dict(Hh=-1), dict(W=-1), dict(C=0),
               dict(heads=0), dict(heads=3), dict(axis=2), dict(axis=-1),
               dict(eps=float("nan")), dict(eps=float("inf")), dict(eps=-1e-5)):
        assert v(hip_lib, **kw) == INVALID, kw


def test_unsupported(hip_lib):
    for kw in (dict(C=128), dict(heads=8), dict(heads=2), dict(W=65),
               dict(Hh=65, axis=COL), dict(B=1 << 40, Hh=1 << 20)):
        assert v(hip_lib, **kw) == UNSUPPORTED, kw
    # only the attended axis is limited
    assert v(hip_lib, Hh=1000, W=32) == OK
    assert v(hip_lib, Hh=32, W=1000, axis=COL) == OK


def test_misaligned(hip_lib):
    for name in ("x", "out", "ln_w", "ln_b", "w_qkv", "w_out"):
        base = {"x": X, "out": OUT, "ln_w": LNW, "ln_b": LNB, "w_qkv": WQKV, "w_out": WOUT}[name]
        assert v(hip_lib, **{name: base + 4}) == MISALIGNED, name
    assert v(hip_lib, b_out=BOUT + 4) == OK
    assert v(hip_lib, b_out=BOUT + 2) == MISALIGNED


def test_overlaps(hip_lib):
    nbytes = 4 * 32 * 32 * 64 * 4
    assert v(hip_lib, out=X + 16) == INVALID            # partial overlap with x
    assert v(hip_lib, out=X + nbytes) == OK              # adjacent
    assert v(hip_lib, w_qkv=OUT + nbytes - 16) == INVALID
    assert v(hip_lib, b_out=OUT) == INVALID
    assert v(hip_lib, ln_w=X) == OK                      # weights may alias the input


def test_empty_is_ok(hip_lib):
    for kw in (dict(B=0), dict(Hh=0), dict(W=0)):
        assert v(hip_lib, x=0, out=0, **kw) == OK, kw


def test_python_wrapper_rejects_before_any_gpu_call(hip_lib):
    x = torch.zeros((1, 2, 3, 64))
    p = (torch.zeros(64), torch.zeros(64), torch.zeros(192, 64), torch.zeros(64, 64),
         torch.zeros(64))
    with pytest.raises(ValueError):
        hip_lib.axial_pass(x, p, ROW)            # CPU tensor
    with pytest.raises(ValueError):
        hip_lib.axial_block(x.double(), p, p)


def test_block_checks_both_passes_before_any_launch(hip_lib):
    """axial_block validates the row pass and the column pass (its second
    weight set, and the column length Hh) before it launches anything."""
    COL_W = [(i + 8) * SZ for i in range(5)]

    def b(x=X, out=OUT, row=(LNW, LNB, WQKV, WOUT, BOUT), col=tuple(COL_W), B=4, Hh=32, W=32,
          C=64, heads=4, eps=1e-5):
        return hip_lib.lib().axial_block(x, out, *row, *col, B, Hh, W, C, heads, eps, None)

    assert b(Hh=65) == UNSUPPORTED          # column length
    assert b(W=65) == UNSUPPORTED           # row length
    assert b(col=(0,) + tuple(COL_W[1:])) == INVALID
    assert b(col=tuple(COL_W[:2]) + (COL_W[2] + 4,) + tuple(COL_W[3:])) == MISALIGNED
    assert b(col=(OUT,) + tuple(COL_W[1:])) == INVALID   # column weights inside out
    assert b(out=X + 16) == INVALID
    assert b(B=0, x=0, out=0) == OK          # empty: nothing launched


def test_in_place_pass_never_splits(hip_lib):
    """A pass with at most 128 sequences splits each over two workgroups that
    both read every token of it; in place (out == x) one half would read
    tokens the other has already overwritten, so the launch must not split."""
    split = hip_lib.axial_pass_split
    # The page's images: 4 x 32 x 32, 128 sequences per pass.
    assert split(X, OUT, 4, 32, 32, ROW) == 2
    assert split(X, OUT, 4, 32, 32, COL) == 2
    assert split(X, X, 4, 32, 32, ROW) == 1
    assert split(X, X, 4, 32, 32, COL) == 1
    # More sequences than half the CUs: never split.
    assert split(X, OUT, 8, 32, 32, ROW) == 1
    assert split(X, OUT, 2, 100, 64, ROW) == 1
    # Every small shape: in place is always 1.
    for B, Hh, W in ((1, 1, 1), (1, 64, 1), (3, 7, 45), (4, 32, 32), (1, 2, 64)):
        for axis in (ROW, COL):
            assert split(X, X, B, Hh, W, axis) == 1
            assert split(X, OUT, B, Hh, W, axis) in (1, 2)
    # Invalid: axis, negative or empty sizes, sequence longer than 64.
    assert split(X, OUT, 4, 32, 32, 2) == -1
    assert split(X, OUT, -1, 32, 32, ROW) == -1
    assert split(X, OUT, 0, 32, 32, ROW) == -1
    assert split(X, OUT, 1, 1, 65, ROW) == -1
    assert split(X, OUT, 1, 65, 1, COL) == -1
