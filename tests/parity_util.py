"""Comparison helpers shared by the GPU parity tests (no kernel arithmetic here)."""
import numpy as np

import oracle

# Tolerance on bf16 outputs: max |y_gpu - y_ref| / rms(y_ref) <= 2e-2 per call.
BF16_TOL = 2e-2
# fp32 layers (fp32 weights and activations, fp32 accumulation on the GPU).
F32_TOL = 1e-4
# Routing ids are compared exactly on every token whose exact gap between the k-th and
# (k+1)-th logit is at least DELTA; inside the window the GPU choice only has to be a
# valid top-k of the exact logits up to DELTA. fp32 logits of a 2048-long dot product of
# bf16 x and N(0, 0.02) weights differ from the exact ones by ~1e-6 (H=128: ~1e-7).
DELTA = {2048: 3e-5, 128: 2e-6}


def rel_err(got, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / rms) if ref.size else 0.0


def delta_for(hidden: int) -> float:
    return DELTA.get(hidden, 3e-5 * np.sqrt(hidden / 2048.0))


def check_routing(layer, x, gpu_ids, gpu_w, delta):
    """Returns the number of tokens inside the tie window (ids may then differ)."""
    ref_ids, ref_w, margin = oracle.route(layer, x)
    z = oracle.logits(layer, x)
    k = layer.top_k
    sure = margin >= delta
    assert np.array_equal(gpu_ids[sure], ref_ids[sure]), "routing ids differ off the tie window"
    assert np.all(np.abs(gpu_w[sure] - ref_w[sure]) <= 1e-5), "routing weights differ"
    assert np.all(np.abs(gpu_w.sum(1) - 1.0) <= 1e-5)
    assert np.all(np.diff(gpu_ids, axis=1) > 0), "ids not strictly ascending"
    for t in np.nonzero(~sure)[0]:
        kth = np.sort(z[t])[::-1][k - 1]
        assert np.all(z[t, gpu_ids[t]] >= kth - delta), f"token {t}: invalid top-k"
    return int((~sure).sum())


def check_grouping(layer, gpu):
    """Grouping is a pure function of the GPU's own ids: compare bit for bit."""
    ids = gpu["topk_ids"]
    counts, offsets, sorted_tok, slot_of = oracle.group(layer, ids)
    assert np.array_equal(gpu["counts"], counts)
    assert np.array_equal(gpu["offsets"], offsets)
    assert np.array_equal(gpu["sorted_tok"], sorted_tok)
    assert np.array_equal(gpu["slot_of"], slot_of)
    assert counts.sum() == layer.top_k * ids.shape[0]


def to_np(buf: dict) -> dict:
    return {k: v.cpu().numpy() for k, v in buf.items()}
