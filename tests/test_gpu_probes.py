"""The bandwidth probes behind the benchmark's measured-ceiling figures: the copy kernel moves
every byte, and the read-only kernel loads every 16-byte vector once (the XOR of its sink words
is the XOR of all 32-bit words of the source), at sizes with ragged tails of its 8-vector steps
and of its grid."""
import numpy as np
import pytest
import torch

from bit_kv_cache_02_amd import kvq

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 4096 + 16, 256 * 8 * 16 * 3 + 32, (64 << 20) + 112])
def test_copy_and_read_probes(nbytes):
    print(f"[probes] {nbytes} bytes", flush=True)
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.zeros_like(src)
    kvq.hbm_copy(src, dst)
    sink = torch.zeros(kvq.HBM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    kvq.hbm_read(src, sink)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().view(np.uint32), host)
    want = np.bitwise_xor.reduce(host)
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == want


def test_read_probe_leaves_unused_sink_words():
    src = torch.ones(1024, dtype=torch.int32, device="cuda")  # 4 KiB: one workgroup
    sink = torch.full((kvq.HBM_READ_SINK_WORDS,), 7, dtype=torch.int32, device="cuda")
    kvq.hbm_read(src, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy()
    assert got[0] == 0  # 1024 ones XOR to 0
    assert (got[1:] == 7).all()


@pytest.mark.parametrize("out_bytes", [4096, 3 * 4096, 4096 * 2049, (16 << 20) + 4096 * 5])
def test_fold4_probe(out_bytes):
    # the 4:1 read:write probe: output vector 256 m + t is the XOR of input vectors
    # 1024 m + t + 256 k, with ragged tails of its two-group steps and of its grid
    print(f"[probes] fold4 {out_bytes} bytes out", flush=True)
    rng = np.random.default_rng(out_bytes)
    host = rng.integers(0, 1 << 32, out_bytes, dtype=np.uint32)  # 4 * out_bytes bytes
    src = torch.from_numpy(host.view(np.int32)).cuda()
    dst = torch.full((out_bytes // 4,), 7, dtype=torch.int32, device="cuda")
    kvq.hbm_fold4(src, dst)
    torch.cuda.synchronize()
    v = host.reshape(-1, 4, 256, 4)  # [group m][k][t][4 words]
    want = v[:, 0] ^ v[:, 1] ^ v[:, 2] ^ v[:, 3]
    assert np.array_equal(dst.cpu().numpy().view(np.uint32).reshape(-1, 256, 4), want)
