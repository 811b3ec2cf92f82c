"""dit_block_forward_noalloc, the entry point for callers that cannot allocate
device memory: the forward with the library-owned static workspace gives the
same bytes as dit_block_forward with a caller workspace (the same kernels run),
on calls in a row where a later call is smaller and runs over the earlier
call's leftovers; it allocates nothing; sizes beyond the static workspace are
refused before anything is enqueued (GPU)."""
import pytest
import torch

from _helpers import bits, run_block
from memory_bounded_chunked_amd import block as B
from memory_bounded_chunked_amd import synth

pytestmark = pytest.mark.gpu

BF16_A = synth.BlockShape("noalloc-bf16-a", 256, 2, 128, 512, 777, "bf16")
BF16_B = synth.BlockShape("noalloc-bf16-b", 256, 2, 128, 512, 300, "bf16")
W8 = synth.BlockShape("noalloc-w8", 256, 2, 128, 512, 611, "w8_bf16")
TINY = synth.CONFIGS["tiny"]


def _noalloc(shape, inputs, ca, cm, fc=0, check_free=True):
    blk, x, mod = B.block_from_inputs(shape, inputs, "cuda")
    need = blk.peak_workspace(shape.n_tokens, ca, cm, fc)
    assert need <= B.STATIC_WORKSPACE_BYTES, need
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    blk.forward_noalloc(x, mod, ca, cm, fc)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == alloc0
    if check_free:
        assert torch.cuda.mem_get_info()[0] == free0
    out = x.cpu()
    blk.close()
    return out


def test_noalloc_matches_caller_workspace_on_calls_in_a_row():
    big = synth.make_inputs(BF16_A, seed=0)
    small = synth.make_inputs(BF16_B, seed=1)
    # the first call on the device may load the library's code (and with it the
    # static buffer), so device free memory is compared from the second call on
    first = _noalloc(BF16_A, big, 256, 256, check_free=False)
    assert bits(first) == bits(run_block(BF16_A, big, 256, 256))
    second = _noalloc(BF16_B, small, 128, 64)
    assert bits(second) == bits(run_block(BF16_B, small, 128, 64))
    # the larger call again, now over the smaller call's leftovers
    assert bits(_noalloc(BF16_A, big, 0, 777)) == bits(first)


def test_noalloc_fp32_and_int8_weights():
    tiny = synth.make_inputs(TINY, seed=0)
    w8 = synth.make_inputs(W8, seed=0)
    a = _noalloc(TINY, tiny, TINY.attn_chunk, TINY.mlp_chunk, check_free=False)
    assert bits(a) == bits(run_block(TINY, tiny, TINY.attn_chunk, TINY.mlp_chunk))
    b = _noalloc(W8, w8, 200, 100, 256)
    assert bits(b) == bits(run_block(W8, w8, 200, 100, 256))


def test_noalloc_refuses_sizes_beyond_the_static_workspace():
    shape = BF16_B
    blk, x, mod = B.block_from_inputs(shape, synth.make_inputs(shape, seed=0), "cuda")
    n_big = 1 << 17  # global K and V alone: 2 * 131072 * 256 * 2 B = 128 MiB
    assert blk.peak_workspace(n_big, 8192, 8192) > B.STATIC_WORKSPACE_BYTES
    before = bits(x.cpu())
    lib = B.load_library()
    rc = lib.dit_block_forward_noalloc(blk._h, x.data_ptr(), mod.data_ptr(), None, None, n_big, 8192, 8192, 0,
                                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == B.DIT_ETOOBIG
    assert "static workspace" in B.strerror(rc)
    assert bits(x.cpu()) == before
    with pytest.raises(B.DitError):
        blk.forward_noalloc(x, mod, 0, 0)  # mlp_chunk_tokens 0: DIT_EINVAL, as for dit_block_forward
    blk.close()
