"""The seeded input generators: shapes and structure of the five workloads
(CPU only; large ones are built without their values)."""
import numpy as np
import pytest

from paged_kv_varlen_flash_amd import workloads as W


def test_tiny_mixed_structure():
    wl = W.make("tiny_mixed")
    assert wl.B == 2 and wl.T == 38 and wl.num_blocks == 16
    assert list(wl.q_lens) == [37, 1] and list(wl.k_lens) == [37, 81]
    assert (wl.block_table[0] >= 0).sum() == 3 and (wl.block_table[1] >= 0).sum() == 6
    used = wl.block_table[wl.block_table >= 0]
    assert len(set(used.tolist())) == 9 and used.max() < 16
    # slot mapping = block_table lookup of each new token's position
    assert wl.slot_mapping[0] == wl.block_table[0, 0] * 16
    assert wl.slot_mapping[37] == wl.block_table[1, 80 // 16] * 16 + 80 % 16
    assert wl.q.shape == (38, 4, 64) and wl.kv_cache.shape == (2, 16, 16, 2, 64)
    # new-token slots hold the sentinel before the scatter
    BS = 16
    for s in wl.slot_mapping:
        assert np.all(wl.kv_cache[:, s // BS, s % BS] == W.SENTINEL)


@pytest.mark.parametrize("name", ["decode_llama8b", "chunked_prefill_mix", "cascade_prefix",
                                  "long_decode_d256"])
def test_large_structure(name):
    wl = W.make(name, materialise=False)
    spec = wl.spec
    assert np.all(wl.q_lens >= 1) and np.all(wl.q_lens <= wl.k_lens)
    nblk = (wl.k_lens + wl.BS - 1) // wl.BS
    for b in range(wl.B):
        assert np.all(wl.block_table[b, :nblk[b]] >= 0)
        assert np.all(wl.block_table[b, nblk[b]:] == -1)
    if spec.shared_prefix:
        P = spec.shared_prefix // wl.BS
        assert np.all(wl.block_table[:, :P] == wl.block_table[0, :P])
        priv = np.concatenate([wl.block_table[b, P:nblk[b]] for b in range(wl.B)])
        assert len(set(priv.tolist())) == len(priv)
        assert not set(priv.tolist()) & set(wl.block_table[0, :P].tolist())
    else:
        allb = np.concatenate([wl.block_table[b, :nblk[b]] for b in range(wl.B)])
        assert len(set(allb.tolist())) == len(allb) == wl.num_blocks
    if name == "decode_llama8b":
        assert wl.B == 64 and np.all(wl.q_lens == 1)
        assert wl.k_lens.min() >= 512 and wl.k_lens.max() <= 4096
    if name == "chunked_prefill_mix":
        pre = wl.q_lens > 1
        assert pre.sum() == 8 and np.all(wl.q_lens[pre] == wl.k_lens[pre])
        assert (~pre).sum() == 56
    if name == "cascade_prefix":
        s = wl.k_lens - 2048
        assert wl.B == 32 and s.min() >= 64 and s.max() <= 512
    if name == "long_decode_d256":
        assert wl.B == 16 and wl.k_lens.min() >= 32768 and wl.k_lens.max() <= 131072


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... 1.015625)
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_regenerate_one_sequence():
    wl = W.make("decode_llama8b", materialise=False)
    only = W.sample_sequences(wl, 3)
    W.materialise_values(wl, only=only)
    full = W.make("decode_llama8b")
    for b in only:
        t = wl.cu_seqlens_q[b]
        assert np.array_equal(wl.q[t], full.q[t])
        nb = (wl.k_lens[b] + 15) // 16
        ids = wl.block_table[b, :nb]
        assert np.array_equal(wl.kv_cache[:, ids], full.kv_cache[:, ids])


def test_prefill_rows_of_the_mix():
    """chunked_prefill_mix_prefill holds exactly the prefill sequences of
    chunked_prefill_mix (same lengths, no decodes)."""
    mix = W.make("chunked_prefill_mix", materialise=False)
    pre = W.make("chunked_prefill_mix_prefill", materialise=False)
    rows = mix.q_lens > 1
    assert np.array_equal(np.sort(mix.q_lens[rows]), np.sort(pre.q_lens))
    assert np.array_equal(np.sort(mix.k_lens[rows]), np.sort(pre.k_lens))
    assert np.array_equal(pre.q_lens, pre.k_lens) and pre.q_lens.size == 8
