"""The byte and flop models bench.py prices its roofline with, checked against the per-unit
figures of the method's measurement contract at d = 128, H = 48, Cch = 3 * 48 * 128 = 18 432,
bf16 inputs: per node and head the verify moves q, k, v, beta, g in (772 B), o out (512 B) and
the k, u, ln g bank (1028 B); per pending token the fold reads 1028 * H + 4 * Cch bytes; the
conv window is read and written (2 * 12 * Cch); the conv weights are 8 * Cch per layer; a
state tile is 4 d^2.  Also: the bench refuses more than one GPU."""
import numpy as np
import pytest

import bench
from gated_deltanet_tree_amd import binding

D, H = 128, 48
CCH = 3 * H * D
TILE = 4 * D * D
BF16 = 2


def _view(sizes):
    """Schedule view of chains of the given node counts (one sequence each)."""
    trees = [np.array([-1] + list(range(n - 1)), dtype=np.int32) for n in sizes]
    return binding.schedule_view(binding.hld_schedule(trees))


def test_per_node_verify_bytes():
    v = _view([7])
    assert bench.ut_bytes(v, [0], H, D, BF16) == H * TILE + 7 * 110_976
    # a folding sequence adds the tile write-back and 1028 B per pending token and head
    assert (bench.ut_bytes(v, [5], H, D, BF16) - bench.ut_bytes(v, [0], H, D, BF16)
            == H * TILE + 5 * 1028 * H)


def test_fused_method_bytes_per_unit():
    v = _view([9])
    base = bench.fused_method_bytes(v, [0], H, D, BF16)
    # per node: conv inputs in (36 864), beta/g (4 B per head), o (512 B per head), the k, u,
    # ln g bank (1028 B per head) and the fp32 conv-input bank (73 728)
    per_node = 36_864 + 4 * H + 512 * H + 1028 * H + 73_728
    # per sequence: the tile read and the conv window read + written; the weights once
    assert base == H * TILE + 442_368 + 9 * per_node + 147_456
    # per pending token: 1028 H + 4 Cch = 123 072 B, plus the tile write-back once
    for L in (1, 3, 8):
        assert bench.fused_method_bytes(v, [L], H, D, BF16) - base == H * TILE + L * 123_072


def test_fused_kernel_bytes_bank_raw_inputs():
    """The kernel's own count banks the bf16 inputs' bits (half the fp32 bank) and reads only
    the last three pending conv rows; with nothing pending it differs from the method model by
    the bank's width and the window write-back."""
    v = _view([9])
    m, k = (f(v, [0], H, D, BF16) for f in (bench.fused_method_bytes, bench.fused_bytes))
    assert m - k == 9 * (73_728 - CCH * BF16) + 12 * CCH
    # folding five tokens: the kernel reads 3 pending conv rows, the model 5 fp32 rows
    m5, k5 = (f(v, [5], H, D, BF16) for f in (bench.fused_method_bytes, bench.fused_bytes))
    assert (m5 - m) - (k5 - k) == 5 * 4 * CCH - (3 * BF16 * CCH + 12 * CCH)


def test_chain_wave_bytes_count_boundary_tiles():
    """One chain of n nodes in one wave: its start tile read and one tile per stored node."""
    v = _view([6])
    assert int(v["n_waves"]) == 1
    stores = int(np.count_nonzero(v["node_store"] >= 0))
    assert (bench.verify_wave_bytes(v, 0, [0], H, D, BF16)
            == H * TILE * (1 + stores) + 6 * 110_976)


def test_prefill_models():
    T, S = 16_384, 8
    assert bench.prefill_bytes(T, S, H, D) == T * H * 1284 + 2 * S * H * TILE
    assert bench.prefill_flops(T, H, D) == 7 * D * D * T * H
    # the split products' ridge against HBM, and the path's intensity below it
    ridge = bench.SPLIT_MATRIX_PEAK_TFLOPS * 1e12 / (bench.HBM_PEAK_GBPS * 1e9)
    assert ridge == pytest.approx(104.17, abs=0.01)
    assert bench.prefill_flops(T, H, D) / bench.prefill_bytes(T, S, H, D) < ridge


def test_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one MI355X" in capsys.readouterr().err


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    """A counter record is tied to the kernel's code: editing a comment or the layout keeps it,
    editing code drops it."""
    import shutil
    for name in bench.KERNEL_SOURCES["prefill"]:
        shutil.copy(f"{bench.CSRC}/{name}", tmp_path / name)
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    h0 = bench.kernel_source_sha256("prefill")
    src = (tmp_path / "prefill.hip").read_text()
    (tmp_path / "prefill.hip").write_text(src.replace("// tokens per chunk", "// chunk length"))
    assert src.count("// tokens per chunk") == 1 and bench.kernel_source_sha256("prefill") == h0
    # a reformat that moves no token keeps it too
    (tmp_path / "prefill.hip").write_text(src.replace("kC = 16;", "kC =\n        16 ;"))
    assert bench.kernel_source_sha256("prefill") == h0
    (tmp_path / "prefill.hip").write_text(src.replace("kC = 16;", "kC = 32;"))
    assert bench.kernel_source_sha256("prefill") != h0
    (tmp_path / "prefill.hip").write_text(src.replace("constexpr int kC", "constexpr intkC"))
    assert bench.kernel_source_sha256("prefill") != h0
