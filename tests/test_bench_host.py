"""Host-side accounting of bench.py (no GPU): effective FLOPs are 4*D times the
legal (b, h, i, j) pairs the oracle counts; algorithmic bytes follow their
definition; the multi-GPU request is refused with a message."""
import numpy as np
import pytest

import bench
import oracle
import workloads as W


@pytest.mark.parametrize("cfg,over", [(1, {}), (2, {}), (3, dict(H=2, Lq=300, Lk=300)),
                                      (5, dict(B=3, H=2)), (4, dict(B=2, H=4, Lq=64, Lk=96))])
def test_effective_flops_are_4d_times_oracle_pairs(cfg, over):
    w = W.config(cfg, **over)
    flops, _, pairs_row = bench.work(w)
    pairs = oracle.unmasked_pairs(w.kind, w.B, w.H, w.Lq, w.Lk, w.lens, w.f64("add"))
    assert flops == 4.0 * w.D * pairs
    assert int(pairs_row.sum()) * w.H == pairs


def test_llama_causal_closed_forms():
    # 32 heads x L(L+1)/2 causal pairs; Q, K, V, O at 16 MiB each
    w = W.config(3)
    flops, alg, _ = bench.work(w)
    assert flops == 4 * 128 * 32 * 2048 * 2049 // 2 == 34_376_515_584
    assert alg == 64 * 2**20


def test_prenorm_cross_closed_forms():
    # no mask: B*H*Lq*Lk pairs; x, K, V, out at 128 MiB each plus gamma and beta
    w = W.config(4)
    flops, alg, _ = bench.work(w)
    assert flops == 4 * 64 * 2**31
    assert alg == 512 * 2**20 + 2 * 1024 * 2


def test_padding_bytes_count_only_used_keys():
    w = W.make("pad", "f16", B=2, H=3, Lq=40, Lk=50, D=16, kind=W.PADDING, seed=1,
               lens_range=(10, 10))
    w.lens = np.array([10, 30], np.int32)
    _, alg, _ = bench.work(w)
    # Q + O for every row, K + V for keys below each length, 4-byte lengths
    assert alg == 2 * 2 * 3 * 40 * 16 * 2 + 2 * (10 + 30) * 3 * 16 * 2 + 4 * 2


def test_multi_gpu_request_exits_with_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_kernel_hash_ignores_comments_only():
    a = 'int f(int x) { return x + 1; }  // one\n/* two */ const char* s = "// kept";'
    b = '/* other words */\nint f(int x) {\n  return x + 1;   // three\n}\nconst char* s = "// kept";'
    c = 'int f(int x) { return x + 2; } const char* s = "// kept";'
    d = 'int f(int x) { return x + 1; } const char* s = "// changed";'
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    assert bench._code_only(a) != bench._code_only(d)


def test_kernel_hash_per_family():
    import os
    csrc = os.path.join(os.path.dirname(bench.__file__), "masked_head_attention_amd", "csrc")
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(csrc, f)), f
        assert len(bench.kernel_source_hash(kernel)) == 16
    assert bench.kernel_source_hash(bench.KERNEL_NAME) != \
        bench.kernel_source_hash(bench.SOFTMAX_KERNEL_NAME)


def test_decode_accounting_matches_the_oracle_pairs():
    """Decode: 4 D FLOPs per legal (key, head) pair, the pairs being those of
    the one-row forward with key padding; bytes are q and out, K and V of the
    legal cache rows, the lengths and the float32 LSE."""
    w = W.decode_config(B=3, H=2, Lk=300, lens_range=(0, 300))
    w.lens = np.array([0, 300, 117], np.int32)
    flops, alg = bench.decode_work(w)
    pairs = oracle.unmasked_pairs(W.PADDING, w.B, w.H, 1, w.Lk, w.lens, None)
    assert pairs == 2 * (0 + 300 + 117)
    assert flops == 4.0 * w.D * pairs
    assert alg == (2 * 3 * 2 * 128 * 2 + 2 * (0 + 300 + 117) * 2 * 128 * 2 + 4 * 3 + 4 * 3 * 2)


def test_decode_workload_closed_form():
    w = W.decode_config()
    flops, alg = bench.decode_work(w)
    assert flops == 4 * 128 * 32 * int(w.lens.sum())
    assert (w.lens >= 256).all() and (w.lens <= 4096).all()


def test_backward_flops_are_ten_d_per_pair():
    # five products of 2 D per legal pair: 2.5 x the forward's 4 D
    w = W.config(W.BWD_CONFIG)
    fwd, _, _ = bench.work(w)
    assert fwd * 10.0 / 4.0 == 10 * 128 * 32 * 2048 * 2049 // 2


def test_grad_output_leaves_the_workload_unchanged():
    a = W.config(1)
    g = W.grad_output(a)
    b = W.config(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert g.shape == (a.B, a.H, a.Lq, a.D) and np.array_equal(g, W.grad_output(b))
