"""CPU checks of the input layouts the GPU tests feed the library: the
flattened (ragged) layout and the scattered-row layout are pure data movement
of the padded batch, so every row they hold must be found where their
offsets and indices say."""
import numpy as np

import workloads as W


def _ragged_batch():
    b = W.generate(W.config(5, N=12, V=96))
    assert b["draft_probs"] is not None
    return b


def _gammas(b):
    ids = b["draft_ids"]
    return np.where((ids < 0).any(axis=1), np.argmax(ids < 0, axis=1), ids.shape[1])


def test_flatten_places_every_row():
    b = _ragged_batch()
    f = W.flatten(b)
    gam = _gammas(b)
    cu = f["cu_num_draft_tokens"]
    np.testing.assert_array_equal(cu, np.cumsum(gam))
    T = int(cu[-1])
    assert f["draft_ids"].shape == (T,) and f["target_logits"].shape[0] == T + len(gam)
    qrow = 0
    for i, g in enumerate(gam):
        lo = cu[i] - g
        np.testing.assert_array_equal(f["draft_ids"][lo:cu[i]], b["draft_ids"][i, :g])
        np.testing.assert_array_equal(f["u_accept"][lo:cu[i]], b["u_accept"][i, :g])
        # request i's target rows start at lo + i: its drafts, then its bonus
        np.testing.assert_array_equal(f["target_logits"][lo + i:cu[i] + i + 1], b["target_logits"][i, :g + 1])
        if f["has_draft_probs"][i]:
            np.testing.assert_array_equal(f["draft_probs"][qrow:qrow + g], b["draft_probs"][i, :g])
            qrow += g
    assert qrow == f["draft_probs"].shape[0]


def test_scatter_rows_indices_name_the_ordered_rows():
    for dtype in ("bf16", "f32"):
        b = W.generate(W.config(2, N=9, V=40, dtype=dtype))
        f = W.flatten(b)
        s = W.scatter_rows(f, 5, 7)
        N = len(f["cu_num_draft_tokens"])
        T = f["draft_ids"].shape[0]
        tl, st = f["target_logits"], s["target_logits"]
        assert st.shape == (T + N + 7, tl.shape[1])
        cu = f["cu_num_draft_tokens"]
        for i in range(N):
            lo = (cu[i - 1] if i else 0)
            for t in range(lo, cu[i]):
                np.testing.assert_array_equal(st[s["target_logits_indices"][t]], tl[t + i])
            np.testing.assert_array_equal(st[s["bonus_logits_indices"][i]], tl[cu[i] + i])
        used = np.concatenate([s["target_logits_indices"], s["bonus_logits_indices"]])
        assert len(np.unique(used)) == T + N
        junk = np.setdiff1d(np.arange(st.shape[0]), used)
        assert len(junk) == 7
        vals = W.bf16_bits_to_f32(st[junk]) if dtype == "bf16" else st[junk]
        assert np.isnan(vals).all()
