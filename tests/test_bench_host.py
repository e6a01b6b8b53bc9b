"""bench.py's host-side arithmetic and refusals, on the CPU (no GPU is touched):
the algorithmic flop and byte counts it divides by, the counter-table
reduction behind the traffic record, and the single-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_causal_flops_convention():
    # 4*B*H*Lq*Lk*D, halved for causal (the usual convention); within 1/L of
    # 4*D times the exact number of visible query-key pairs
    assert bench.causal_flops(1, 32, 8192, 8192, 128, False) == 4.0 * 32 * 8192 * 8192 * 128
    assert bench.causal_flops(1, 32, 8192, 8192, 128, True) == 5.4975581388800e11
    for L in (64, 200, 1000):
        exact = 4.0 * 128 * int(oracle.allowed_mask(L, L, True, -1).sum())
        assert abs(bench.causal_flops(1, 1, L, L, 128, True) - exact) <= exact / L


@pytest.mark.parametrize("Lq,Lk,W,causal", [(10, 10, 3, True), (10, 10, 3, False), (7, 20, 5, True),
                                            (20, 7, 2, False), (33, 33, 0, True), (5, 9, 100, False)])
def test_window_pairs_match_the_mask(Lq, Lk, W, causal):
    assert bench.window_pairs(Lq, Lk, W, causal) == int(oracle.allowed_mask(Lq, Lk, causal, W).sum())


def test_decode_bytes_formula():
    ctx = np.array([1, 16, 17, 4096, 600])
    Hq, Hkv, D = 12, 2, 128
    kv = int(ctx.sum()) * Hkv * D * 2 * 2            # K and V, once per KV head
    q_out = len(ctx) * Hq * D * 2 * 2                # q read, out written
    lse = len(ctx) * Hq * 4
    table = 4 * int(sum((c + 15) // 16 for c in ctx))
    assert bench.decode_bytes(ctx, Hq, Hkv, D) == kv + q_out + lse + table + 4 * len(ctx)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for d, name, value in rows:
            f.write(f'{d},"{name}","{counter}",{value}\n')


def test_traffic_record_reduction(tmp_path, monkeypatch):
    out = tmp_path / "record.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    calib = "void at::native::vectorized_elementwise_kernel<4, mul>"
    fwd = "void attn::fwd_kernel<attn::BF16, 128, false, false>(attn::FwdArgs)"
    split = "void attn::decode_split_kernel<attn::BF16, 128>(attn::DecArgs)"
    comb = "void attn::decode_combine_kernel<attn::BF16, 128>(attn::DecArgs)"
    fill = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>>"
    # FETCH_SIZE reads half the true bytes on the multiply; per-dispatch values
    # split over two rows (two channels) must be summed per dispatch
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(1, fill, 7.0), (2, calib, 131072.0), (2, calib, 131072.0),
                  (3, fwd, 50000.0), (3, fwd, 25000.0), (4, fwd, 74000.0), (5, split, 76000.0), (6, comb, 1900.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(1, calib, 524288.0), (2, fwd, 66560.0), (3, split, 3450.0), (4, comb, 200.0)])
    bench.write_traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), ["test"])
    rec = {}
    for line in out.read_text().splitlines():
        if ":" in line and not line.startswith(("#", " ")):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    assert float(rec["fetch_scale"]) == pytest.approx(2.0)
    assert float(rec["fetch_bytes_per_launch"]) == pytest.approx(74500.0 * 1024 * 2.0, rel=1e-6)
    assert float(rec["decode_split_fetch_bytes_per_launch"]) == pytest.approx(76000.0 * 1024 * 2.0, rel=1e-6)
    assert float(rec["write_scale"]) == pytest.approx(1.0)
    assert float(rec["write_bytes_per_launch"]) == pytest.approx(66560.0 * 1024, rel=1e-6)
    # the record is read back only while the forward's sources are unchanged
    assert bench.traffic_record() == {"workload": "gqa8k_causal", "fetch_bytes": pytest.approx(74500.0 * 1024 * 2.0),
                                      "write_bytes": pytest.approx(66560.0 * 1024)}
    monkeypatch.setattr(bench, "FWD_SOURCES", bench.FWD_SOURCES[:1])
    assert bench.traffic_record() is None
