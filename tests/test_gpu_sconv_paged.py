"""GPU parity of inkattn_sconv_paged: the sconv state kept in a paged cache
(the K/V cache of a virtual sliding-window layer of window 3), against the
oracle's convolution of whole sequences; chunked calls, prefix blocks shared
between sequences, and bitwise equality with the dense-state kernel."""

import numpy as np
import pytest
import torch

import attention_sconv_amd as ink
from attention_sconv_amd import kvcache
import oracle
import synth
from gpu_util import ddtype, dev, host, idev

pytestmark = pytest.mark.gpu


def _close(got, want, dtype, what):
    if dtype == "fp32":
        assert np.abs(got - want).max() <= 1e-5, what
    else:
        err = np.abs(got - want)
        assert (err <= np.abs(want) * 2.0 ** -8 + 1e-5).all(), f"{what}: {err.max()}"


class Paged:
    """A KV cache and a paged state cache with random block tables."""

    def __init__(self, dtype, H, lengths, rng, extra=3, shared=None):
        self.dtype, self.H, self.C = dtype, H, H * 128
        nb = [(L + 127) // 128 for L in lengths]
        self.nblocks = sum(nb) + extra
        perm = rng.permutation(self.nblocks).astype(np.int32)
        self.bt = np.zeros((len(lengths), max(nb)), np.int32)
        k = 0
        for b, n in enumerate(nb):
            self.bt[b, :n] = perm[k:k + n]
            k += n
        if shared is not None:                      # (dst seq, src seq, blocks)
            dst, src, nshared = shared
            self.bt[dst, :nshared] = self.bt[src, :nshared]
        self.sbt = self.bt.copy()                   # the state layer uses the same tables
        td = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.kc, self.vc = kvcache.alloc(self.nblocks, H, dtype)
        self.kc.fill_(float("nan"))
        self.vc.fill_(float("nan"))
        self.ks = torch.full((self.nblocks, 128, self.C), float("nan"), dtype=td, device="cuda")
        self.vs = torch.full_like(self.ks, float("nan"))

    def call(self, k_in, v_in, w, seqs_chunks):
        """seqs_chunks: list of (seq b, first position, n tokens); k_in/v_in rows packed."""
        cu = np.zeros(len(seqs_chunks) + 1, np.int32)
        for i, (_, _, n) in enumerate(seqs_chunks):
            cu[i + 1] = cu[i] + n
        seq_lens = np.array([p + n for (_, p, n) in seqs_chunks], np.int32)
        slots = np.concatenate([oracle.slots_for(self.bt[b], np.arange(p, p + n))
                                for (b, p, n) in seqs_chunks]).astype(np.int32)
        sbt = np.stack([self.sbt[b] for (b, _, _) in seqs_chunks])
        ink.inkattn_sconv_paged(ddtype(self.dtype), self.H, 128, len(seqs_chunks), int(cu[-1]),
                                int(max(n for (_, _, n) in seqs_chunks)), dev(k_in, self.dtype),
                                dev(v_in, self.dtype), dev(w, self.dtype), idev(cu),
                                idev(seq_lens), idev(sbt), self.ks, self.vs, idev(slots),
                                self.kc, self.vc)

    def outputs(self, b, L):
        slots = oracle.slots_for(self.bt[b], np.arange(L)).astype(np.int64)
        k, v = kvcache.slots_of(self.kc, self.vc, slots)
        return host(k).reshape(L, self.C), host(v).reshape(L, self.C)


def _draw(rng, shape, dtype, std=1.0):
    a = (rng.standard_normal(shape) * std).astype(np.float32)
    return synth.round_bf16(a) if dtype == "bf16" else a


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sconv_paged_chunks_equal_whole_sequences(dtype):
    rng = np.random.default_rng(100)
    H = 4
    lengths = [300, 129, 5, 256]
    chunks = [[100, 1, 199], [128, 1], [1, 1, 3], [3, 253]]       # per sequence, in order
    pg = Paged(dtype, H, lengths, rng)
    w = _draw(rng, (2, H * 128, 4), dtype, 0.5)
    xk = [_draw(rng, (L, H * 128), dtype) for L in lengths]
    xv = [_draw(rng, (L, H * 128), dtype) for L in lengths]
    pos = [0] * len(lengths)
    for step in range(max(len(c) for c in chunks)):
        calls, ks, vs = [], [], []
        for b, c in enumerate(chunks):
            if step < len(c):
                calls.append((b, pos[b], c[step]))
                ks.append(xk[b][pos[b]:pos[b] + c[step]])
                vs.append(xv[b][pos[b]:pos[b] + c[step]])
                pos[b] += c[step]
        pg.call(np.concatenate(ks), np.concatenate(vs), w, calls)
    torch.cuda.synchronize()
    for b, L in enumerate(lengths):
        k, v = pg.outputs(b, L)
        yk, _ = oracle.sconv_sequence(xk[b], w[0])
        yv, _ = oracle.sconv_sequence(xv[b], w[1])
        _close(k, yk, dtype, f"k seq {b}")
        _close(v, yv, dtype, f"v seq {b}")
        # the state cache holds the inputs, bit for bit
        rows = oracle.slots_for(pg.sbt[b], np.arange(L))
        ks_rows = host(pg.ks.reshape(-1, H * 128)[torch.from_numpy(rows).cuda()])
        np.testing.assert_array_equal(ks_rows, xk[b].astype(np.float64))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_sconv_paged_shared_prefix_blocks(dtype):
    # sequence 1 reuses the first two state (and K/V) blocks of sequence 0:
    # its first new token's halo is positions 253..255 of the shared prefix
    rng = np.random.default_rng(101)
    H = 2
    pg = Paged(dtype, H, [300, 260], rng, shared=(1, 0, 2))
    w = _draw(rng, (2, H * 128, 4), dtype, 0.5)
    pk = _draw(rng, (256, H * 128), dtype)
    pv = _draw(rng, (256, H * 128), dtype)
    a_k, a_v = _draw(rng, (44, H * 128), dtype), _draw(rng, (44, H * 128), dtype)
    b_k, b_v = _draw(rng, (4, H * 128), dtype), _draw(rng, (4, H * 128), dtype)
    pg.call(pk, pv, w, [(0, 0, 256)])                                # the prefix, once
    pg.call(np.concatenate([a_k, b_k]), np.concatenate([a_v, b_v]), w,
            [(0, 256, 44), (1, 256, 4)])
    torch.cuda.synchronize()
    for b, (sk, sv) in enumerate([(a_k, a_v), (b_k, b_v)]):
        L = 256 + len(sk)
        k, v = pg.outputs(b, L)
        yk, _ = oracle.sconv_sequence(np.concatenate([pk, sk]), w[0])
        yv, _ = oracle.sconv_sequence(np.concatenate([pv, sv]), w[1])
        _close(k, yk, dtype, f"k seq {b}")
        _close(v, yv, dtype, f"v seq {b}")


def test_sconv_paged_equals_dense_state_bitwise():
    # a chunk after 37 context tokens: the dense kernel gets the last three
    # context rows as its state, the paged one finds them in the state cache
    rng = np.random.default_rng(102)
    H, ctx, n = 4, 37, 90
    dtype = "bf16"
    w = _draw(rng, (2, H * 128, 4), dtype, 0.5)
    hk, hv = _draw(rng, (ctx, H * 128), dtype), _draw(rng, (ctx, H * 128), dtype)
    xk, xv = _draw(rng, (n, H * 128), dtype), _draw(rng, (n, H * 128), dtype)
    pg = Paged(dtype, H, [ctx + n], rng)
    pg.call(hk, hv, w, [(0, 0, ctx)])
    pg.call(xk, xv, w, [(0, ctx, n)])
    kc, vc = kvcache.alloc(pg.nblocks, H, dtype)
    state = np.stack([np.stack([hk[-3:], hv[-3:]])])                # [1][2][3][C]
    slots = oracle.slots_for(pg.bt[0], np.arange(ctx, ctx + n)).astype(np.int32)
    st = dev(state, dtype)
    ink.inkattn_sconv(ddtype(dtype), H, 128, 1, n, n, dev(xk, dtype), dev(xv, dtype),
                      dev(w, dtype), st, idev(np.zeros(1, np.int32)),
                      idev(np.array([0, n], np.int32)), idev(slots), kc, vc)
    torch.cuda.synchronize()
    sl = torch.from_numpy(slots.astype(np.int64)).cuda()
    k1, v1 = kvcache.slots_of(pg.kc, pg.vc, sl)
    k2, v2 = kvcache.slots_of(kc, vc, sl)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
