"""GPU parity: libfa.so (through the C ABI) against the fp64 oracle on the same
seeded inputs.  Tolerances: max relative L2 error 1e-5 for fp32 inputs, 2e-2
for bf16 and 5e-3 for fp16 inputs (fp32 accumulation), per output tensor."""
import numpy as np
import pytest
import torch

import workloads as wl
from harness import (TOL, compare, device_inputs, gpu_groups, kv_heads_complete, oracle_groups, run_gpu,
                     run_oracle, say)

pytestmark = pytest.mark.gpu

F32, BF16, F16 = torch.float32, torch.bfloat16, torch.float16

# small cases spanning several tiles, ragged tails and the degenerate situations
EDGE_CASES = {
    "cross_attn_nomask": dict(lens_q=[5, 130, 64], lens_kv=[70, 33, 200], head_num=4, kv_heads=2, head_dim=64,
                              sparse_mode=0),
    "rdcausal_lq_gt_lkv": dict(lens_q=[150, 40], lens_kv=[60, 40], head_num=2, kv_heads=1, head_dim=128,
                               sparse_mode=3),
    "lucausal_lq_ne_lkv": dict(lens_q=[90, 200], lens_kv=[300, 65], head_num=2, kv_heads=2, head_dim=128,
                               sparse_mode=2),
    "band_gqa": dict(lens_q=[300, 129, 1], head_num=6, kv_heads=3, head_dim=128, sparse_mode=4, pre_tokens=37,
                     next_tokens=11),
    "band_neg_pre": dict(lens_q=[257, 64], head_num=2, kv_heads=2, head_dim=64, sparse_mode=4, pre_tokens=-5,
                         next_tokens=40),
    "zero_length_seqs": dict(lens_q=[0, 77, 0, 150], lens_kv=[10, 77, 0, 150], head_num=3, kv_heads=1,
                             head_dim=128, sparse_mode=3),
    "all_features": dict(lens_q=[37, 200, 129], head_num=4, kv_heads=2, head_dim=128, sparse_mode=3,
                         keep_prob=0.8, alibi=True, sink=True),
    "d64_causal_varlen": dict(lens_q=[33, 513, 128], head_num=8, kv_heads=2, head_dim=64, sparse_mode=3),
    "single_tokens": dict(lens_q=[1, 1, 2], head_num=2, kv_heads=1, head_dim=128, sparse_mode=3, sink=True),
    "sink_dropout_band": dict(lens_q=[190, 67], head_num=2, kv_heads=1, head_dim=64, sparse_mode=4,
                              pre_tokens=50, next_tokens=3, keep_prob=0.7, sink=True),
    # prefix (mode 6): N in [Lkv - Lq, Lkv] (Lq <= Lkv) or [0, Lkv] (Lq > Lkv)
    "prefix_varlen": dict(lens_q=[200, 77, 129, 5], lens_kv=[300, 40, 129, 64], head_num=4, kv_heads=2,
                          head_dim=128, sparse_mode=6, prefix=[150, 17, 64, 60]),
    "prefix_edges_sink_dropout": dict(lens_q=[190, 67, 300], head_num=2, kv_heads=1, head_dim=64, sparse_mode=6,
                                      prefix=[0, 67, 299], keep_prob=0.8, sink=True),
    "prefix_alibi": dict(lens_q=[150, 300], head_num=4, kv_heads=1, head_dim=128, sparse_mode=6,
                         prefix=[30, 129], alibi=True),
    # attenMask [S1Max, S2Max] (1 = masked out), shared by the sequences at their local indices
    "mask_mode1_varlen": dict(lens_q=[200, 77, 129], lens_kv=[130, 300, 129], head_num=4, kv_heads=2,
                              head_dim=128, sparse_mode=1, mask=(0.3, [5, 100])),
    "mask_band_drop_sink": dict(lens_q=[190, 67], head_num=2, kv_heads=1, head_dim=64, sparse_mode=4,
                                pre_tokens=50, next_tokens=3, keep_prob=0.8, sink=True, mask=(0.2, [])),
    "mask_mode0_alibi_gqa": dict(lens_q=[150, 300], head_num=4, kv_heads=1, head_dim=128, sparse_mode=0,
                                 alibi=True, mask=(0.5, [7])),
    # generated pse: pseType 3 (square-root distance) and [B, N] slopes
    "pse_sqrt_causal_gqa": dict(lens_q=[150, 300, 37], head_num=4, kv_heads=2, head_dim=128, sparse_mode=3,
                                alibi=True, pse_type=3),
    "pse_sqrt_batch_slopes_drop_sink": dict(lens_q=[190, 67, 129], head_num=2, kv_heads=1, head_dim=64,
                                            sparse_mode=2, alibi=True, pse_type=3, slopes_per_batch=True,
                                            keep_prob=0.8, sink=True),
    "alibi_batch_slopes_band": dict(lens_q=[257, 64], head_num=4, kv_heads=4, head_dim=128, sparse_mode=4,
                                    pre_tokens=40, next_tokens=0, alibi=True, slopes_per_batch=True),
    "cross_nomask_d128": dict(lens_q=[200, 77, 129], lens_kv=[130, 300, 129], head_num=4, kv_heads=2,
                              head_dim=128, sparse_mode=0),
    # head dims the kernels pad (to 128 and to 64)
    "d96_causal_drop_sink": dict(lens_q=[150, 67, 300], head_num=4, kv_heads=2, head_dim=96, sparse_mode=3,
                                 keep_prob=0.85, sink=True),
    "d32_band_alibi": dict(lens_q=[200, 129], head_num=2, kv_heads=1, head_dim=32, sparse_mode=4, pre_tokens=40,
                           next_tokens=5, alibi=True),
    "d80_cross": dict(lens_q=[90, 200], lens_kv=[300, 65], head_num=2, kv_heads=2, head_dim=80, sparse_mode=0),
    # external pse (pseType 1: before scaling, 0: after): full block, one shared row, 1024-row compression
    "pse_full_type1_cross": dict(lens_q=[200, 77, 129], lens_kv=[130, 300, 129], head_num=4, kv_heads=2,
                                 head_dim=128, sparse_mode=0, pse=("full", False), pse_type=1),
    "pse_row_type0_drop_sink": dict(lens_q=[190, 67], head_num=2, kv_heads=1, head_dim=64, sparse_mode=3,
                                    pse=("row", True), pse_type=0, keep_prob=0.8, sink=True),
    "pse_compressed_causal": dict(lens_q=[1100, 300], head_num=2, kv_heads=2, head_dim=64, sparse_mode=3,
                                  pse=("compressed", False), pse_type=1),
    # sparse modes 7 / 8: the band on the last / first sequence, a causal triangle on the others
    "mode7_varlen_drop_sink": dict(lens_q=[200, 77, 300], lens_kv=[260, 77, 450], head_num=4, kv_heads=2,
                                   head_dim=128, sparse_mode=7, pre_tokens=100, next_tokens=8, keep_prob=0.85,
                                   sink=True),
    # a chunk split off a 400-token sequence (rows 250..399 against keys 0..399), global alibi positions
    "mode8_split_alibi_sink": dict(lens_q=[150, 129, 64], lens_kv=[400, 129, 64], head_num=4, kv_heads=1,
                                   head_dim=128, sparse_mode=8, pre_tokens=180, next_tokens=0, alibi=True,
                                   sink=True, q_start_idx=250, kv_start_idx=0),
    # value head dim below the query / key one (qD == kD >= vD), on zero-padded copies
    "vd64_qd128_causal_drop_sink": dict(lens_q=[150, 67, 300], head_num=4, kv_heads=2, head_dim=128,
                                        v_head_dim=64, sparse_mode=3, keep_prob=0.85, sink=True),
    "vd32_qd96_band_alibi": dict(lens_q=[200, 129], head_num=2, kv_heads=1, head_dim=96, v_head_dim=32,
                                 sparse_mode=4, pre_tokens=40, next_tokens=5, alibi=True),
    "vd80_qd128_cross": dict(lens_q=[90, 200], lens_kv=[300, 65], head_num=2, kv_heads=2, head_dim=128,
                             v_head_dim=80, sparse_mode=0),
    "mode8_sqrt_d64_drop": dict(lens_q=[300, 40, 1], head_num=2, kv_heads=2, head_dim=64, sparse_mode=8,
                                pre_tokens=64, next_tokens=16, alibi=True, pse_type=3, keep_prob=0.9,
                                q_start_idx=1000, kv_start_idx=1000),
}


def _edge(name, dtype, seed):
    kw = dict(EDGE_CASES[name])
    lq = kw.pop("lens_q")
    lkv = kw.pop("lens_kv", None)
    if "mask" in kw:
        p_masked, full_rows = kw.pop("mask")
        kw["atten_mask"] = wl.random_atten_mask(seed, max(lq), max(lkv or lq), p_masked, full_rows)
    return wl.make_case(name, lq, lkv, dtype=dtype, seed=seed, **kw)


@pytest.mark.parametrize("deterministic", [True, False])
@pytest.mark.parametrize("dtype", [F32, BF16, F16])
@pytest.mark.parametrize("name", list(EDGE_CASES))
def test_edge_case(name, dtype, deterministic):
    if "pse" in EDGE_CASES[name] and dtype != F32:
        pytest.skip("kept off the device: a bf16 run of these cases faulted in the fused 16-bit external-pse "
                    "kernels (no longer built; cause not shown). 16-bit external pse now runs the "
                    "materialised-score path, covered by test_gpu_pse16.py")
    seed = 100 + list(EDGE_CASES).index(name)
    case = _edge(name, dtype, seed)
    say(f"edge {name} dtype={dtype} det={deterministic} seed={seed} lens={list(case.lens_q)}/{list(case.lens_kv)}")
    gpu = run_gpu(case, deterministic)
    ref = run_oracle(case)
    compare(gpu, ref, TOL[dtype], case=case)


@pytest.mark.parametrize("deterministic", [True, False])
def test_workload1_fp32_full(deterministic):
    case = wl.make_workload(1)
    say(f"workload 1 full det={deterministic}")
    compare(run_gpu(case, deterministic), run_oracle(case), TOL[F32], case=case)


@pytest.fixture(scope="module")
def workload2():
    return wl.make_workload(2)


@pytest.fixture(scope="module")
def workload2_oracle(workload2):
    # every sequence (lengths 1736, 630, 337, 701, 922, 1692, 994, 304) and every head
    return oracle_groups(workload2, range(workload2.kv_heads))


@pytest.mark.parametrize("deterministic", [True, False])
def test_workload2_every_sequence(workload2, workload2_oracle, deterministic):
    case = workload2
    say(f"workload 2 det={deterministic}: all {case.batch} sequences, all {case.head_num} heads")
    gpu = gpu_groups(run_gpu(case, deterministic), case, range(case.kv_heads))
    compare(gpu, workload2_oracle, TOL[BF16], case=case)


def test_deterministic_is_bitwise_reproducible(workload2):
    case = workload2
    say("workload 2 determinism")
    x = device_inputs(case)
    a = run_gpu(case, True, inputs=x)
    b = run_gpu(case, True, inputs=x)
    for key in ("out", "m", "l", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key


def test_deterministic_bitwise_with_dropout_and_alibi():
    case = wl.make_workload(4)
    say("workload 4 determinism")
    x = device_inputs(case)
    runs = [run_gpu(case, True, inputs=x) for _ in range(3)]
    for key in ("out", "m", "l", "dq", "dk", "dv"):
        for r in runs[1:]:
            assert np.array_equal(runs[0][key], r[key]), key


def test_dropout_keep_bits_bit_exact():
    # Q = 0 makes every allowed logit equal, and V = I maps key j to column j, so
    # O[i, j] = z_ij / (keep * n_i): its non-zero pattern is the keep bits.
    lens = [37, 128, 101]
    keep = 0.6
    case = wl.make_case("dropout_probe", lens, head_num=2, kv_heads=1, head_dim=128, dtype=BF16, keep_prob=keep,
                        seed=7)
    case.q.zero_()
    v = torch.zeros_like(case.v)
    for b in range(len(lens)):
        s = int(case.cu_seqlens_kv[b])
        for j in range(lens[b]):
            v[s + j, 0, j] = 1.0
    case.v = v
    say("dropout bit-exact probe")
    gpu = run_gpu(case, True, backward=False)
    bits = np.unpackbits(case.drop_mask, bitorder="little")
    off = 0
    for b, L in enumerate(lens):
        s = int(case.cu_seqlens_q[b])
        for h in range(2):
            z = bits[off:off + L * L].reshape(L, L).astype(bool)
            off += L * L
            got = gpu["out"][s:s + L, h, :L] != 0
            assert np.array_equal(got, z), (b, h)


@pytest.mark.parametrize("deterministic", [True, False])
def test_workload3_sampled_heads(deterministic):
    case = wl.make_workload(3)
    batches, heads = [0], [0, 21]
    say(f"workload 3 det={deterministic} batches={batches} heads={heads}")
    gpu = run_gpu(case, deterministic)
    ref = run_oracle(case, batches=batches, heads=heads)
    compare(gpu, ref, TOL[BF16], kv_select=kv_heads_complete(case, heads), case=case)


@pytest.mark.parametrize("deterministic", [True, False])
def test_workload4_sampled_heads(deterministic):
    case = wl.make_workload(4)
    batches, heads = [0, 15], [0, 9]
    say(f"workload 4 det={deterministic} batches={batches} heads={heads}")
    gpu = run_gpu(case, deterministic)
    ref = run_oracle(case, batches=batches, heads=heads)
    compare(gpu, ref, TOL[BF16], kv_select=kv_heads_complete(case, heads), case=case)


@pytest.fixture(scope="module")
def workload5():
    say("generating workload 5")
    return wl.make_workload(5)


def test_workload5_kv_group_against_oracle(workload5):
    # The timed workload in the benchmark's launch configuration; one whole kv group (8 query
    # heads, all 64 sequences including the 16,384-token one) against the oracle: O, max, sum,
    # dQ of the group's heads, dK/dV of its kv head, and dSink of its heads summed over every
    # sequence.  The groups share every sequence and run the same kernel paths.
    case = workload5
    g = 3
    G = case.head_num // case.kv_heads
    heads = list(range(g * G, (g + 1) * G))
    say(f"workload 5: kv group {g} (heads {heads[0]}-{heads[-1]}), all {case.batch} sequences, "
        f"longest {int(case.lens_q.max())}")
    gpu = run_gpu(case, True, heads=heads, kv_heads=[g])
    ref = oracle_groups(case, [g])
    compare(gpu, ref, TOL[BF16], case=case)


def test_workload5_dsink_identity_every_head(workload5):
    # dSink of all 64 heads: -sum_i exp(sink_h - m_i) / l_i * rowsum(dY * O) in fp64 from the
    # device's own O, m, l (the group test above checks those, and dSink, against the oracle)
    case = workload5
    say("workload 5 dsink identity")
    gpu = run_gpu(case, True)
    dy = case.dy.double().numpy()
    delta = np.einsum("tnd,tnd->tn", dy, gpu["out"])
    p_sink = np.exp(case.sink.astype(np.float64)[None, :] - gpu["m"]) / gpu["l"]
    expect = -(p_sink * delta).sum(axis=0)
    err = np.linalg.norm(gpu["dsink"] - expect) / np.linalg.norm(expect)
    say(f"dsink identity relL2={err:.2e}")
    assert err <= TOL[BF16]


@pytest.mark.parametrize("deterministic", [True, False])
def test_workload4_fp16_sampled_heads(deterministic):
    # dropout + alibi at full size in fp16 (the atomic D = 128 path routes alibi to the deterministic passes)
    case = wl.make_workload(4, F16)
    batches, heads = [3], [1, 14]
    say(f"workload 4 fp16 det={deterministic} batches={batches} heads={heads}")
    gpu = run_gpu(case, deterministic)
    ref = run_oracle(case, batches=batches, heads=heads)
    compare(gpu, ref, TOL[F16], kv_select=kv_heads_complete(case, heads), case=case)


def test_workload5_fp16_longest_shortest_median():
    # the timed workload in fp16, in the launch configuration the benchmark times: kv group 6
    # on the longest (16,384), shortest and median sequences against the oracle
    case = wl.make_workload(5, F16)
    lens = case.lens_q
    order = np.argsort(lens)
    batches = [int(order[-1]), int(order[0]), int(order[len(order) // 2])]
    g = 6
    G = case.head_num // case.kv_heads
    say(f"workload 5 fp16 group {g} batches={batches} lens={[int(lens[b]) for b in batches]}")
    gpu = run_gpu(case, True, heads=list(range(g * G, (g + 1) * G)), kv_heads=[g])
    ref = oracle_groups(case, [g], batches=batches)
    # dSink sums over every sequence: the three chosen ones do not make it
    compare(gpu, ref, TOL[F16], keys=("out", "m", "l", "dq", "dk", "dv"), case=case)
