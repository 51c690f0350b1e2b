"""The Python binding rejects wrong caller buffers before any pointer reaches
the library (CPU only).

The kernels write through lse, out, dq/dk/dv and the workspace without
bounds, so a short or mistyped buffer must raise in the binding.  Without a
GPU here, the tensors are stand-ins that carry exactly the attributes the
binding reads (shape, dtype, device, layout, pointer); the library call
itself is replaced by one that fails the test if it is ever reached.
"""

import pytest
import torch

import io_aware_tiled_05_amd as fa


class Dev:
    def __init__(self, i=0):
        self.i = i

    def __eq__(self, o):
        return isinstance(o, Dev) and o.i == self.i

    def __hash__(self):
        return self.i


class T:
    """A stand-in for a device tensor."""

    def __init__(self, shape, dtype=torch.bfloat16, dev=0, contiguous=True, cuda=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = Dev(dev)
        self.is_cuda = cuda
        self._contig = contiguous

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def contiguous(self):
        return self

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()

    def data_ptr(self):
        return 4096


B, H, N, D = 2, 3, 100, 64


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    def refuse(*a, **k):
        raise AssertionError("a bad buffer reached the library")
    monkeypatch.setattr(fa, "_call", refuse)
    monkeypatch.setattr(fa, "fa_bwd_workspace_size", lambda B, H, N, d: 4096)
    monkeypatch.setattr(fa, "fa_decode_workspace_size", lambda B, H, Nq, Nk, d: 4096)


def qkv():
    return T((B, H, N, D)), T((B, H, N, D)), T((B, H, N, D))


GOOD_LSE = dict(shape=(B, H, N), dtype=torch.float32)
BAD_LSE = {
    "short": T((B, H, N - 1), torch.float32),
    "bf16": T((B, H, N), torch.bfloat16),
    "other_gpu": T((B, H, N), torch.float32, dev=1),
    "strided": T((B, H, N), torch.float32, contiguous=False),
    "host": T((B, H, N), torch.float32, cuda=False),
}
BAD_OUT = {
    "short": T((B, H, N - 1, D)),
    "fp16": T((B, H, N, D), torch.float16),
    "other_gpu": T((B, H, N, D), dev=1),
    "strided": T((B, H, N, D), contiguous=False),
}


@pytest.mark.parametrize("bad", sorted(BAD_LSE))
def test_forward_rejects_bad_lse(bad):
    q, k, v = qkv()
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd(q, k, v, out=T((B, H, N, D)), lse=BAD_LSE[bad])
    bm = T((1, 1), torch.uint8)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd_blocksparse(q, k, v, bm, out=T((B, H, N, D)), lse=BAD_LSE[bad])
    with pytest.raises(ValueError, match="lse"):
        fa.fa_fwd_dropout(q, k, v, 0.1, 1, out=T((B, H, N, D)), lse=BAD_LSE[bad])


@pytest.mark.parametrize("bad", sorted(BAD_OUT))
def test_forward_rejects_bad_out(bad):
    q, k, v = qkv()
    lse = T(**GOOD_LSE)
    with pytest.raises(ValueError):
        fa.fa_fwd(q, k, v, out=BAD_OUT[bad], lse=lse)
    with pytest.raises(ValueError):
        fa.fa_fwd_blocksparse(q, k, v, T((1, 1), torch.uint8), out=BAD_OUT[bad], lse=lse)


@pytest.mark.parametrize("bad", sorted(BAD_LSE))
def test_backward_rejects_bad_lse(bad):
    q, k, v = qkv()
    o, dO = T((B, H, N, D)), T((B, H, N, D))
    g = [T((B, H, N, D)) for _ in range(3)]
    ws = T((1024,), torch.float32)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd(q, k, v, o, BAD_LSE[bad], dO, dq=g[0], dk=g[1], dv=g[2], workspace=ws)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd_noalloc(q, k, v, o, BAD_LSE[bad], dO, *g)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_bwd_stage(fa.FA_BWD_STAGE_D, q, k, v, o, BAD_LSE[bad], dO, *g, ws)


@pytest.mark.parametrize("which", [0, 1, 2])
@pytest.mark.parametrize("bad", sorted(BAD_OUT))
def test_backward_rejects_bad_gradient_buffers(which, bad):
    q, k, v = qkv()
    o, dO, lse = T((B, H, N, D)), T((B, H, N, D)), T(**GOOD_LSE)
    g = [T((B, H, N, D)) for _ in range(3)]
    g[which] = BAD_OUT[bad]
    ws = T((1024,), torch.float32)
    with pytest.raises(ValueError):
        fa.fa_bwd(q, k, v, o, lse, dO, dq=g[0], dk=g[1], dv=g[2], workspace=ws)
    with pytest.raises(ValueError):
        fa.fa_bwd_blocksparse(q, k, v, o, lse, dO, T((1, 1), torch.uint8), dq=g[0], dk=g[1],
                              dv=g[2], workspace=ws)
    with pytest.raises(ValueError):
        fa.fa_bwd_noalloc(q, k, v, o, lse, dO, *g)


def test_backward_rejects_short_workspace():
    q, k, v = qkv()
    o, dO, lse = T((B, H, N, D)), T((B, H, N, D)), T(**GOOD_LSE)
    g = [T((B, H, N, D)) for _ in range(3)]
    short = T((1023,), torch.float32)  # 4092 bytes of the 4096 needed
    with pytest.raises(ValueError, match="workspace"):
        fa.fa_bwd(q, k, v, o, lse, dO, dq=g[0], dk=g[1], dv=g[2], workspace=short)
    with pytest.raises(ValueError, match="workspace"):
        fa.fa_bwd_stage(fa.FA_BWD_STAGE_D, q, k, v, o, lse, dO, *g, short)
    with pytest.raises(ValueError, match="workspace"):
        fa.fa_bwd(q, k, v, o, lse, dO, dq=g[0], dk=g[1], dv=g[2],
                  workspace=T((1024,), torch.float32, dev=1))


def test_decode_rejects_bad_out_and_lse():
    q = T((B, H, 1, D))
    k, v = T((B, H, 50, D)), T((B, H, 50, D))
    ws = T((1024,), torch.float32)
    with pytest.raises(ValueError):
        fa.fa_decode(q, k, v, out=T((B, H, 2, D)), lse=T((B, H, 1), torch.float32), workspace=ws)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_decode(q, k, v, out=T((B, H, 1, D)), lse=T((B, H, 50), torch.float32),
                     workspace=ws)
    with pytest.raises(ValueError, match="workspace"):
        fa.fa_decode(q, k, v, out=T((B, H, 1, D)), lse=T((B, H, 1), torch.float32),
                     workspace=T((10,), torch.float32))


def test_block_mask_and_key_len_checked():
    q, k, v = qkv()
    out, lse = T((B, H, N, D)), T(**GOOD_LSE)
    with pytest.raises(ValueError, match="block_mask"):
        fa.fa_fwd_blocksparse(q, k, v, T((2, 2), torch.uint8), out=out, lse=lse)  # nb = 1
    with pytest.raises(ValueError, match="key_len"):
        fa.fa_fwd(q, k, v, key_len=T((B + 1,), torch.int32), out=out, lse=lse)
    with pytest.raises(ValueError, match="key_len"):
        fa.fa_fwd(q, k, v, key_len=T((B,), torch.int64), out=out, lse=lse)


def test_noalloc_refuses_strided_key_len():
    q, k, v = qkv()
    o, dO, lse = T((B, H, N, D)), T((B, H, N, D)), T(**GOOD_LSE)
    g = [T((B, H, N, D)) for _ in range(3)]
    with pytest.raises(ValueError, match="key_len"):
        fa.fa_bwd_noalloc(q, k, v, o, lse, dO, *g, key_len=T((B,), torch.int32, contiguous=False))
