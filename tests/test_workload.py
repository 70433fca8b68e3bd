"""Properties of the seeded input generators (CPU only)."""
import numpy as np
import pytest

import workload


@pytest.mark.parametrize("name", sorted(workload.WORKLOADS))
def test_structure(name):
    w = workload.WORKLOADS[name](structure_only=True)
    bs = w.block_size
    n_needed = -(-w.context_lens // bs)
    used = set()
    for b in range(w.B):
        ids = w.block_tables[b, :n_needed[b]]
        assert ids.min() >= 0 and ids.max() < w.N_blocks
        assert (w.block_tables[b, n_needed[b]:] == w.poison_block).all()
        used.update(int(i) for i in ids)
    assert w.poison_block not in used
    assert w.N_blocks == -(-11 * len(used) // 10) or name in ("tiny_fp32", "tinylm_mha_bf16")
    assert w.context_lens.min() >= w.T
    assert n_needed.max() <= w.max_blocks


def test_length_ranges():
    assert list(workload.tiny_fp32(structure_only=True).context_lens) == [37, 100]
    c2 = workload.tinylm_mha_bf16(structure_only=True).context_lens
    assert c2.min() >= 1 and c2.max() <= 512
    c3 = workload.llama1b_gqa_append(structure_only=True)
    assert c3.lens_pre.min() >= 128 and c3.lens_pre.max() <= 4096
    assert (c3.context_lens == c3.lens_pre + 1).all() and c3.max_blocks == 257
    c4 = workload.llama8b_prefix_share(structure_only=True).context_lens
    assert c4.min() >= 16 and c4.max() <= 8192
    assert 700 < np.median(c4) < 1400
    c5 = workload.longctx_verify(structure_only=True).context_lens
    assert c5.min() >= 16384 and c5.max() <= 65536
    pf = workload.llama8b_chunked_prefill(structure_only=True)
    assert pf.T == 512 and (pf.context_lens == pf.lens_pre + 512).all()
    assert pf.lens_pre.min() >= 0 and pf.lens_pre.max() <= 3584 and pf.max_blocks == 256
    lp = workload.llama8b_long_prompt_chunk(structure_only=True)
    assert lp.B == 1 and lp.T == 512 and list(lp.lens_pre) == [8192] and list(lp.context_lens) == [8704]
    assert lp.max_blocks == 544


def test_private_blocks_are_not_shared():
    w = workload.llama1b_gqa_append(structure_only=True)
    n = -(-w.context_lens // 16)
    ids = np.concatenate([w.block_tables[b, :n[b]] for b in range(w.B)])
    assert len(ids) == len(set(ids.tolist()))


def test_prefix_sharing_structure():
    w = workload.llama8b_prefix_share(structure_only=True)
    n = -(-w.context_lens // 16)
    for g in range(16):
        members = range(16 * g, 16 * g + 16)
        longest = max(members, key=lambda b: n[b])
        for b in members:
            k = min(n[b], 32)
            assert (w.block_tables[b, :k] == w.block_tables[longest, :k]).all()
        own = np.concatenate([w.block_tables[b, 32:n[b]] for b in members])
        assert len(own) == len(set(own.tolist()))
    prefix_sets = [set(w.block_tables[16 * g, :min(n[16 * g], 32)].tolist()) for g in range(16)]
    for a in range(16):
        for c in range(a + 1, 16):
            assert not prefix_sets[a] & prefix_sets[c]


def test_poison_marks_unreadable_slots_only():
    w = workload.tinylm_mha_bf16()
    vals = w.values(w.k_pool)
    for b in range(w.B):
        L = int(w.context_lens[b])
        n = -(-L // 16)
        rows = vals[w.block_tables[b, :n]].reshape(n * 16, w.Hkv, w.D)
        assert np.isfinite(rows[:L]).all()
        assert np.isnan(rows[L:]).all()
    assert np.isnan(vals[w.poison_block]).all()


def test_append_slots_poisoned_until_written():
    w = workload.llama1b_gqa_append()
    vals = w.values(w.k_pool[:, :, :1, :4])
    for b in range(0, w.B, 7):
        pos = int(w.lens_pre[b])
        assert np.isnan(vals[w.block_tables[b, pos // 16], pos % 16]).all()
        assert np.isfinite(vals[w.block_tables[b, (pos - 1) // 16], (pos - 1) % 16]).all()


def test_seeded_reproducible_and_bf16_exact():
    a = workload.tinylm_mha_bf16()
    b = workload.tinylm_mha_bf16()
    assert (a.k_pool == b.k_pool).all() and (a.q == b.q).all()
    v = a.values(a.q)
    assert (workload.f32_to_bf16_bits(v) == a.q).all()


def test_relabel_keeps_logical_rows():
    w = workload.tinylm_mha_bf16()
    w2 = workload.relabel_physical(w, seed=5)
    for b in range(w.B):
        n = -(-int(w.context_lens[b]) // 16)
        assert (w.k_pool[w.block_tables[b, :n]] == w2.k_pool[w2.block_tables[b, :n]]).all()
