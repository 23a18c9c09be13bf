"""The benchmark's algorithmic work per launch (CPU only): the byte and flop
counts that its roofline divides by, against sizes worked out by hand from the
workload shapes."""
import bench
import workloads as W


def test_prefill_causal_pairs_and_flops():
    wl = W.WORKLOADS["prefill_q4096_n131072"]
    # queries at positions 126976 .. 131071 (one sequence): sum of (pos + 1)
    assert bench.causal_pairs(wl) == sum(range(126977, 131073)) == 528_484_352
    assert bench.score_flops(wl) == 528_484_352 * 32 * 128 * 2


def test_decode_bytes():
    wl = W.WORKLOADS["decode_b64_n131072"]
    assert bench.score_bytes(wl, False) == 64 * 131072 * 256 + 64 * (32 * 128 * 2 + 32 * 4)
    wl8 = W.WORKLOADS["decode_b8_n1048576_fp8"]
    assert bench.score_bytes(wl8, True) == 8 * (1 << 20) * 132 + 8 * (32 * 128 + 32 * 4 + 32 * 4)
    assert bench.topk_bytes(wl) == 64 * 131072 * 4 + 64 * 2048 * 4
    assert bench.mla_bytes(wl) == 64 * (2048 * 1152 + 2048 * 4 + 64 * 576 * 2 + 64 * 512 * 4)


def test_roofline_bound_follows_arithmetic_intensity():
    pre = W.WORKLOADS["prefill_q4096_n131072"]
    r = bench.roofline("indexer_score", pre, False, bench.score_bytes(pre, False), 3.5, 1)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["achieved"] - bench.score_flops(pre) / 3.5e-3 / 1e12) < 0.1
    pre8 = W.WORKLOADS["prefill_q4096_n131072_fp8"]
    assert bench.roofline("indexer_score", pre8, True, bench.score_bytes(pre8, True), 2.0, 1)["peak"] == 5000.0
    dec = W.WORKLOADS["decode_b64_n131072"]
    r = bench.roofline("indexer_score", dec, False, 2 * bench.score_bytes(dec, False), 0.8, 2)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - 2 * bench.score_bytes(dec, False) / 0.8e-3 / 1e9) < 0.1
    assert r["bytes_per_launch"] == bench.score_bytes(dec, False)
    r = bench.roofline("topk", pre, False, bench.topk_bytes(pre), 1.8, 1)
    assert r["bound"] == "hbm"


def test_fp8_latent_bytes():
    wl = W.WORKLOADS["decode_b64_n131072_kv8"]
    assert bench.mla_bytes(wl) == 64 * (2048 * 656 + 2048 * 4 + 64 * 576 * 2 + 64 * 512 * 4)


def test_score_and_topk_without_a_buffer():
    # one gsa_indexer_topk call moves the score's inputs and writes the indices;
    # at prefill its matrix work decides the bound as for the score alone
    dec = W.WORKLOADS["decode_b8_n1048576_fp8"]
    assert bench.launch_bytes("indexer_topk", dec, True) == bench.score_bytes(dec, True) + 8 * 2048 * 4
    pre = W.WORKLOADS["prefill_q4096_n131072"]
    r = bench.roofline("indexer_topk", pre, False, bench.launch_bytes("indexer_topk", pre, False), 6.0, 1)
    assert r["bound"] == "mfma" and r["kernel"] == "indexer_topk"


def test_step_bytes_match_the_per_query_accounting():
    # per query of a 1 F + 3 S decode group: keys (pos + 1) x 256 B (bf16) or
    # x 132 B (fp8 + scale), q + w, the 8 KiB index write, and per layer
    # 2048 x 1152 B gathered + 8 KiB of indices + 73,728 B of q + 128 KiB of output
    per_layer = 2048 * 1152 + 8192 + 73_728 + 131_072
    assert per_layer == 2_572_288
    dec = W.WORKLOADS["decode_b64_n131072"]
    assert bench.step_bytes(dec, 1, 4) == 64 * (131072 * 256 + 8320 + 8192 + 4 * per_layer) == 2_807_046_144
    m1 = W.WORKLOADS["decode_b8_n1048576_fp8"]
    assert bench.step_bytes(m1, 1, 4) == 8 * ((1 << 20) * 132 + 4352 + 8192 + 4 * per_layer) == 1_189_709_824
    st = W.WORKLOADS["stack78_b8_q8_n262144"]
    # 21 full layers read each sequence's keys once (its 8 queries share them); 78 attention layers
    want = 21 * (8 * (1 << 18) * 256 + 64 * (8320 + 8192)) + 78 * 64 * per_layer
    assert bench.step_bytes(st, 21, 78) == want
    assert abs(want / 8e12 * 1e3 - 3.017) < 0.001          # the stack's 3.017 ms roofline


def test_step_roofline_bounds():
    m1 = W.WORKLOADS["decode_b8_n1048576_fp8"]
    r = bench.step_roofline(m1, True, 1, 4, 0.248)
    assert r["bound"] == "hbm" and abs(r["frac"] - 1_189_709_824 / 0.248e-3 / 8e12) < 1e-4
    pre = W.WORKLOADS["prefill_q4096_n131072_fp8"]
    r = bench.step_roofline(pre, True, 1, 0, 2.0)
    assert r["bound"] == "mfma" and r["peak"] == 5000.0
    assert abs(r["achieved"] - 528_484_352 * 32 * 128 * 2 / 2e-3 / 1e12) < 0.1
