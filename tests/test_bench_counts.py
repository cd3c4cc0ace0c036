"""The bench's algorithmic counts (the roofline's numerator) against the
formulas written out here: per token-head, 10 C d + 6 d^2 flop for tokens of
chunked sequences and 10 C d + 4 d^2 for tokens of tree chunks (sequences of at
most C = 64 tokens, no exit update), with C = 64 and d = d_k = d_v; bytes are
q, k, v, beta and log_gate read once, the initial states read once, and the
requested outputs, states and pseudo-values written once."""
import numpy as np

import bench
from tree_forked_gated_amd import workloads as W


def test_counts_of_the_chain_workload():
    wl = W.chains()
    c = bench.algorithmic_counts(wl, n_out=wl.T, n_state=wl.n_seq, keep_pseudo=False)
    T, H, d, C = 4 * 4096, 16, 128, 64
    assert c["flops"] == T * H * (10 * C * d + 6 * d * d) == 47_244_640_256
    inputs = T * H * (3 * d + 2) * 2          # bf16 q, k, v, beta, log_gate
    init = 4 * H * d * d * 4                  # fp32 initial states
    outs = T * H * d * 2 + 4 * H * d * d * 4  # bf16 outputs, fp32 final states
    assert c["bytes"] == inputs + init + outs == 277_872_640


def test_counts_of_the_draft_tree_workload():
    wl = W.draft_trees()
    c = bench.algorithmic_counts(wl, n_out=wl.T, n_state=0, keep_pseudo=True)
    T, H, d, C = 64 * 64, 32, 128, 64
    assert c["flops"] == T * H * (10 * C * d + 4 * d * d)  # 147,456 per token-head
    inputs = T * H * (3 * d + 2) * 2
    init = 64 * H * d * d * 4
    outs = T * H * d * 2 + T * H * d * 4      # bf16 outputs, fp32 pseudo-values
    assert c["bytes"] == inputs + init + outs == 336_068_608
    # commit: S_0 read and S_a written per path, plus the path's pseudo-values, keys and gates
    cc = bench.commit_counts(wl)
    L = int(wl.path_ptr[-1])
    n_path = wl.n_path
    expect = n_path * H * d * d * 4 * 2 + L * H * (d * 4 + d * 2 + 2) + 4 * (L + 2 * n_path + 1)
    assert cc["bytes"] == expect


def test_tree_and_chain_tokens_split_by_sequence_length():
    """A stream mixing a 64-token tree (no exit update) and a 65-token chain."""
    rng = np.random.default_rng(0)
    par = np.concatenate([W.random_draft_tree(rng, 64), np.arange(-1, 64, dtype=np.int32) + 64]).astype(np.int32)
    par[64] = -1
    seq_start = np.array([0, 64, 129], dtype=np.int32)
    H, d = 2, 128
    q, k, v, beta, g = W._values(rng, 129, H, d, d, "bf16")
    wl = W.Workload("mix", "bf16", par, seq_start, q, k, v, beta, g, W._init(rng, 2, H, d, d, False), None,
                    np.zeros(0, dtype=np.int32))
    c = bench.algorithmic_counts(wl, n_out=129, n_state=0, keep_pseudo=False)
    assert c["flops"] == H * (64 * (10 * 64 * d + 4 * d * d) + 65 * (10 * 64 * d + 6 * d * d))


def test_walk_digest_ignores_comments_only():
    """The traffic counters are keyed by the walk's code: a comment or a blank
    line leaves the key alone, a changed statement does not."""
    import bench
    src = "int a = 1;  // one\n\n// a note\n  int b = a + 2;\n"
    assert bench._code_only(src) == "int a = 1;\nint b = a + 2;"
    assert bench._code_only(src.replace("// a note", "// another note\n\n")) == bench._code_only(src)
    assert bench._code_only(src.replace("a + 2", "a + 3")) != bench._code_only(src)
    assert len(bench.source_digest()) == 16


def test_counter_summaries_are_keyed_by_their_kernel(tmp_path):
    """A counter summary's figures are read only while its digest names the
    current code of its own kernel file: the walk's key is the per-file digest
    of walk_pipe.hip, a summary with another digest gives None, and one whose
    digest matches gives its figure."""
    import bench
    assert bench.source_digest() == bench.kernel_digest("walk_pipe.hip")
    assert len({bench.kernel_digest(f) for f in ("walk_pipe.hip", "chain.hip", "attention.hip")}) == 3
    (tmp_path / "x.md").write_text(f"# x\n\n- source_digest: `{bench.kernel_digest('chain.hip')}`\n- bytes: 123\n")
    (tmp_path / "y.md").write_text("# y\n\n- source_digest: `0000000000000000`\n- bytes: 123\n")
    d = str(tmp_path)
    assert bench.profile_value("x.md", "chain.hip", "bytes", d) == 123.0
    assert bench.profile_value("x.md", "attention.hip", "bytes", d) is None
    assert bench.profile_value("y.md", "chain.hip", "bytes", d) is None
    assert bench.profile_value("missing.md", "chain.hip", "bytes", d) is None
