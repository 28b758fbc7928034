"""The measurement aid gt_calib_gather on the GPU, through the C ABI: its
checksum is the XOR, over the edges, of every 32-bit word of rows K[u] and
V[u] (computed here with numpy), so each edge's rows were read whole; for the
three row sizes it takes, on a ragged edge count, and on the power-law graph
at full size."""
import numpy as np
import pytest
import torch

import gtgen
import sparse_graph_attention_amd as gt
from tests.test_gpu_parity import dev, say, workload

pytestmark = pytest.mark.gpu


def expected(indices, K, V):
    kw = K.reshape(K.shape[0], -1).view(np.uint32)
    vw = V.reshape(V.shape[0], -1).view(np.uint32)
    rows = np.bitwise_xor.reduce(kw, axis=1) ^ np.bitwise_xor.reduce(vw, axis=1)
    return int(np.bitwise_xor.reduce(rows[indices])) if len(indices) else 0


def run(indices, K, V):
    d = dev()
    t = [torch.from_numpy(x).to(d) for x in (indices, K.view(np.int32), V.view(np.int32))]
    c = gt.gt_calib_gather(*t)
    torch.cuda.synchronize()
    return int(c.cpu().numpy().view(np.uint32)[0])


@pytest.mark.parametrize("H,D,dtype", [(8, 32, gtgen.BF16), (8, 32, gtgen.F32), (8, 64, gtgen.F32)])
@pytest.mark.parametrize("E", [1, 1000, 4097 * 3 + 5])
def test_checksum(H, D, dtype, E):
    N = 300
    _, K, V = gtgen.make_features(N, H, D, dtype, 3, 1.0)
    idx = np.random.default_rng(E).integers(0, N, E, dtype=np.int32)
    say("calib H=%d D=%d dtype=%d E=%d" % (H, D, dtype, E))
    assert run(idx, K, V) == expected(idx, K, V)


def test_checksum_powerlaw():
    w = workload("powerlaw")
    say("calib powerlaw")
    assert run(w["indices"], w["K"], w["V"]) == expected(w["indices"], w["K"], w["V"])
