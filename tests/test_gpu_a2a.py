"""GPU parity of the emulated Ulysses all-to-all (bit-exact: it moves data)
against the oracle's per-rank message exchange."""
import numpy as np
import pytest
import torch

import cpinputs
import sequence_context_parallelism_amd as cp
from gpu_util import DEV
from oracle import schedule as Z

pytestmark = pytest.mark.gpu

CASES = [  # S, h, d, sp, dtype
    (256, 32, 128, 4, torch.bfloat16),     # query heads of a 32/8 layer at SP=4
    (256, 8, 128, 4, torch.bfloat16),      # its KV heads
    (192, 2, 64, 8, torch.bfloat16),       # KV replication: 8 ranks, 2 KV heads
    (96, 8, 64, 2, torch.float32),
    (64, 4, 128, 4, torch.float32),        # one head per rank
]


def _host(t):
    return t.cpu().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


@pytest.mark.parametrize("S,h,d,sp,dtype", CASES)
def test_tokens_to_heads_every_rank(gpu_lib, S, h, d, sp, dtype):
    (x,) = cpinputs.normal_torch(7000 + S + h, [(S, h + 2, d)], DEV, dtype)
    xs = x[:, 1:1 + h]                        # strided input: a head window of a wider tensor
    shards = np.split(_host(xs.contiguous()), sp)
    h_out = h // sp if h % sp == 0 else 1
    for r in range(sp):
        y = torch.full((S, h_out, d), -1, device=DEV, dtype=dtype)
        cp.cp_a2a_tokens_to_heads(xs, sp, r, y)
        torch.cuda.synchronize()
        assert np.array_equal(_host(y), Z.a2a_tokens_to_heads(shards, r)), f"rank {r}"


@pytest.mark.parametrize("S,h,d,sp,dtype", [c for c in CASES if c[1] % c[3] == 0])
def test_heads_to_tokens_assembles_every_shard(gpu_lib, S, h, d, sp, dtype):
    outs = cpinputs.normal_torch(8000 + S, [(S, h // sp, d)] * sp, DEV, dtype)
    z = torch.full((S, h + 1, d), -1, device=DEV, dtype=dtype)
    zs = z[:, :h]
    for r in range(sp):
        cp.cp_a2a_heads_to_tokens(outs[r], sp, r, zs)
    torch.cuda.synchronize()
    host_outs = [_host(o) for o in outs]
    zh = _host(zs.contiguous())
    n = S // sp
    for j in range(sp):
        assert np.array_equal(zh[j * n:(j + 1) * n], Z.a2a_heads_to_tokens(host_outs, j)), f"shard {j}"
    assert np.all(_host(z[:, h]) == _host(torch.full((1,), -1, dtype=dtype))[0])   # untouched column


def test_a2a_argument_errors(gpu_lib):
    x = torch.zeros(64, 6, 64, device=DEV, dtype=torch.bfloat16)
    y = torch.zeros(64, 2, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(cp.CpError):
        cp.cp_a2a_tokens_to_heads(x, 4, 0, y)          # 6 heads, 4 ranks
    with pytest.raises(cp.CpError):
        cp.cp_a2a_tokens_to_heads(x[:63], 2, 0, y)     # S not a multiple of... 63 % 2
    with pytest.raises(cp.CpError):
        cp.cp_a2a_tokens_to_heads(x, 3, 3, y)          # rank out of range
