"""Host logic of bench.py, no GPU: the work and byte models against the figures stated for the
causal N=8192 workload, the visible-pair counts of the window and block-sparse workloads against
explicit element masks, the counter-summary parsing, and the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

def test_c3_work_and_bytes():
    # flops: two N x N x d products per head, 2 flops per multiply-add, half of them causal
    assert bench.fwd_flops(2, 16, 8192, 128, True) == 549755813888.0
    assert bench.fwd_flops(2, 16, 8192, 128, False) == 2 * 549755813888.0
    assert bench.bwd_flops(2, 16, 8192, 128, True) == 2.5 * 549755813888.0
    # Q, K, V, O bf16 (64 MiB each) and the fp32 LSE (1 MiB)
    assert bench.fwd_bytes_compulsory(2, 16, 16, 8192, 128) == 4 * 64 * 2**20 + 2**20 == 269484032
    # read Q, K, V, O, dO and LSE; D and the base-2 LSE written and read; fp32 dQ, dK, dV
    assert bench.bwd_bytes_compulsory(2, 16, 16, 8192, 128) == \
        5 * 64 * 2**20 + 2**20 + 4 * 2**20 + 3 * 128 * 2**20 == 743440384
    # the foils: score traffic of naive attention, and tiles re-read per 128-row query tile
    assert bench.naive_bytes(2, 16, 8192) == 17179869184
    assert bench.noreuse_tiled_bytes(2, 16, 8192, 128, causal=True) == 4429185024


def test_grouped_heads_count_kv_once_per_kv_head():
    full = bench.fwd_bytes_compulsory(4, 32, 32, 1024, 128)
    gqa = bench.fwd_bytes_compulsory(4, 32, 8, 1024, 128)
    assert full - gqa == 2 * 4 * (32 - 8) * 1024 * 128 * 2   # K and V of the 24 absent kv-heads


def test_backward_kernel_bytes_cover_the_whole_backward():
    k = bench.bwd_kernel_bytes_compulsory(2, 16, 16, 4096, 128)
    q = 2 * 16 * 4096 * 128
    assert k["bwd_prep"] == 2 * q * 2 + 3 * 2 * 16 * 4096 * 4
    assert k["bwd_dq"] - k["bwd_dkdv"] == q * 4 - 2 * q * 4   # dQ writes one fp32 tensor, dK/dV two


def brute_window(N, left, right, L):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = np.broadcast_to(j < L, (N, N)).copy()
    if left >= 0:
        vis &= j >= i - left
    if right >= 0:
        vis &= j <= i + right
    return int(vis.sum())


@pytest.mark.parametrize("left,right", [(3, 3), (0, 0), (5, -1), (-1, 2), (-1, -1), (40, 7), (0, 100)])
def test_window_pairs_match_an_explicit_mask(left, right):
    N = 37
    assert bench.window_pairs(N, left, right) == brute_window(N, left, right, N)
    lens = np.array([37, 20, 0, 1])
    assert bench.window_pairs(N, left, right, key_lens=lens, B=4) == \
        sum(brute_window(N, left, right, int(L)) for L in lens)


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_pairs_match_the_expanded_bitmap(causal):
    N, bq, bk = 300, 128, 64
    rng = np.random.default_rng(5)
    bm = (rng.random((-(-N // bq), -(-N // bk))) < 0.5).astype(np.uint8)
    el = np.kron(bm, np.ones((bq, bk), dtype=np.uint8))[:N, :N].astype(bool)
    if causal:
        el &= np.tril(np.ones((N, N), dtype=bool))
    assert bench.sparse_pairs(N, bm, causal) == int(el.sum())


def test_stored_traffic_reads_its_row_and_rejects_changed_sources(tmp_path, monkeypatch):
    h = bench._src_hash(bench.KERNEL_SRC["fwd_bf16"])
    f = tmp_path / "hbm_traffic_x.md"
    f.write_text("| Kernel | Sources | a | b | c | Bytes |\n|---|---|---|---|---|---|\n"
                 f"| fwd_bf16 | {h} | 1 | 2 | 3 | 294923658 |\n"
                 "| bwd_dq | 0000000000000000 | 1 | 2 | 3 | 447434710 |\n")
    monkeypatch.setattr(bench, "traffic_file", lambda w: str(f))
    assert bench.stored_traffic("fwd_bf16", "x") == 294923658
    assert bench.stored_traffic("bwd_dq", "x") is None      # sources changed since measured
    assert bench.stored_traffic("bwd_dkdv", "x") is None    # not measured


def test_counter_means_group_dispatches_by_kernel(tmp_path):
    f = tmp_path / "c.csv"
    f.write_text("Kernel_Name,Counter_Value\n"
                 '"void fa::fwd_bf16_kernel<128, true, 1>(fa::FwdParams)",10\n'
                 '"void fa::fwd_bf16_kernel<128, true, 1>(fa::FwdParams)",30\n'
                 '"void fa::bwd_dkdv_kernel<128, true>(fa::BwdParams)",7\n'
                 "__amd_rocclr_copyBuffer,100\n"
                 "some_other_kernel,1\n")
    assert bench._counter_means(str(f)) == {"fwd_bf16": 20.0, "bwd_dkdv": 7.0, "copy": 100.0}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_causal_pairs_with_key_lengths():
    import numpy as np
    for N, L in ((10, 10), (10, 4), (7, 0), (300, 151)):
        i, j = np.arange(N)[:, None], np.arange(N)[None, :]
        assert bench.causal_pairs(N, L) == int(((j <= i) & (j < L)).sum())
    assert bench.causal_pairs(8, 8) == 8 * 9 // 2


def test_every_kernel_source_the_traffic_guard_hashes_exists():
    """The stored counter rows are tied to these files: a missing one would silently change the
    hash rather than fail."""
    for kernel, files in bench.KERNEL_SRC.items():
        for f in files:
            assert os.path.isfile(os.path.join(ROOT, f)), (kernel, f)
