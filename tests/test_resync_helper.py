"""The re-synchronising greedy comparison of the GPU tests (the O-9 parity rule:
a token may differ only at an oracle near-tie; the GPU then restarts from the
oracle's prefix), checked with scripted generators on the CPU."""
import numpy as np
import pytest

from gpu_util import check_greedy_with_resync


def _logits(ref, V, ties):
    """Oracle logits whose choice at k is ref[k], with ref[k] + 1 close behind at the near-ties."""
    z = np.zeros((len(ref), V))
    for k, t in enumerate(ref):
        z[k, t] = 1.0
        z[k, t + 1] = 1.0 - (1e-3 if k in ties else 0.5)
    return z


def _scripted(ref, flips):
    """A generator that follows ref but, when started at or before position k in
    flips, emits ref[k] + 1 at k (as a near-tie could)."""
    calls = []

    def gen(prefix, n):
        start = len(prefix) - 4
        calls.append(start)
        out = list(ref[start:start + n])
        for k in flips:
            if start <= k < start + n:
                out[k - start] += 1
                break
        return out
    return gen, calls


def test_resync_counts_near_ties_and_restarts_from_the_oracle_prefix():
    prompt = [0, 1, 2, 3]
    ref = list(range(10, 30))
    z = _logits(ref, 50, ties={5, 12})
    gen, calls = _scripted(ref, flips=[5, 12])
    assert check_greedy_with_resync(gen, prompt, ref, z) == 2
    assert calls == [0, 6, 13]


def test_resync_rejects_a_mismatch_that_is_not_a_near_tie():
    prompt = [0, 1, 2, 3]
    ref = list(range(10, 30))
    z = _logits(ref, 50, ties={5})
    gen, _ = _scripted(ref, flips=[7])
    with pytest.raises(AssertionError):
        check_greedy_with_resync(gen, prompt, ref, z)


def _scripted_sampled(ref, near_rows):
    """Oracle runs that emit ref from any prefix one token per iteration, with one decision per iteration
    whose margin is 1e-3 at the positions in near_rows (else 0.5)."""
    def oracle_run(prefix, n):
        start = len(prefix) - 4
        toks = list(ref[start:start + n])
        dec = [[("sample", 0, 1e-3 if start + i in near_rows else 0.5)] for i in range(n)]
        return toks, {"emitted": [1] * (n - 1), "decisions": dec}
    return oracle_run


def test_sampled_resync_excuses_only_near_decisions():
    from gpu_util import check_sampled_with_resync
    prompt = [0, 1, 2, 3]
    ref = list(range(10, 30))
    gen, calls = _scripted(ref, flips=[5, 12])
    assert check_sampled_with_resync(gen, _scripted_sampled(ref, {5, 12}), prompt, len(ref)) == 2
    assert calls == [0, 6, 13]
    gen, _ = _scripted(ref, flips=[7])
    with pytest.raises(AssertionError):
        check_sampled_with_resync(gen, _scripted_sampled(ref, {5}), prompt, len(ref))
