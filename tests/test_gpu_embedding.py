"""GPU parity of the embedding (det_embedding): the gather forward and the
table gradient against the oracle, bitwise invariance of dE across every
layout, and the canonical order EDO-v1 bit for bit against the oracle's
FP32 emulation.  Token ids follow a Zipf law, so frequent tokens span many
64-occurrence blocks and most of the vocabulary does not occur."""
import numpy as np
import pytest
import torch

import oracle
from invariant_rmsnorm_backward_amd import adapters, binding, contract, harness, inputs, layouts

pytestmark = pytest.mark.gpu
CONTRACT = contract.load_contract()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "the gpu tests need an MI355X"
    binding.load()


def _wl(name, dim, vocab, lengths, pad_rows=0):
    return inputs.scaled(inputs.workload_embedding(), name, hidden=dim, lengths=lengths,
                         pad_rows=pad_rows, vocab=vocab)


def _reference(wl, data):
    tb = inputs.bf16_bits(data.table.cpu())
    dyb = inputs.bf16_bits(data.dy.cpu())
    dE, dEa = oracle.embedding_bwd_bf16(data.ids, dyb, wl.vocab)
    return {"dE": dE, "y": oracle.embedding_fwd_bf16(data.ids, tb)}, dEa


CASES = {
    "v500_d136": (136, 500, [300, 257, 150], 100),
    "v64_d512_hot": (512, 64, [900, 400], 128),
    "v3000_d8": (8, 3000, [77, 60], 17),
    "v1000_d4096": (4096, 1000, [333, 211], 64),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_embedding_parity_invariance_and_canonical_order(case):
    dim, vocab, lengths, chunk = CASES[case]
    wl = _wl(f"emb_{case}", dim, vocab, lengths)
    data = adapters.make_embedding_inputs(wl, device="cuda", gen_device="cpu")
    ref, dEa = _reference(wl, data)
    cells = layouts.standard_matrix(wl, chunk)
    print(f"[embedding] {case}: {len(cells)} cells, most frequent token "
          f"{np.bincount(data.ids).max()} times", flush=True)
    rep = harness.assert_gradient_batch_invariant("embedding", cells, CONTRACT, data=data,
                                                  reference=ref, raise_on_red=False)
    if not rep.strict:
        print(rep.to_json()[:3000], flush=True)
    assert rep.strict, rep.first_failure
    out = adapters.EmbeddingAdapter().run_cell(cells[0], data)
    # the forward is a copy: bit for bit
    assert np.array_equal(harness.bf16_bits_to_f32(out["y"]).astype(np.float64), ref["y"])
    # EDO-v1 bit for bit against the FP32 emulation
    want = oracle.edo_v1_f32(data.ids, inputs.bf16_bits(data.dy.cpu()), vocab)
    assert np.array_equal(out["dE"].view(np.uint32), want.view(np.uint32))
    absent = np.bincount(data.ids, minlength=vocab) == 0
    assert np.all(out["dE"][absent] == 0) and absent.any()


def test_embedding_padding_rows_are_never_read():
    wl = _wl("emb_pad", 64, 200, [100, 60, 31], pad_rows=40)
    data = adapters.make_embedding_inputs(wl, device="cuda", gen_device="cpu")
    ref, _ = _reference(wl, data)
    cells = [layouts.full(wl), layouts.packed_with_padding(wl), layouts.padded(wl, 230, "left")]
    rep = harness.assert_gradient_batch_invariant("embedding", cells, CONTRACT, data=data,
                                                  reference=ref, raise_on_red=False)
    assert rep.strict, rep.first_failure
    out = adapters.EmbeddingAdapter().run_cell(cells[1], data)
    assert bool(out["pad_rows_clean"][0])


def test_embedding_accumulator_protocol_and_new_ids():
    wl = _wl("emb_proto", 64, 50, [100])
    data = adapters.make_embedding_inputs(wl, device="cuda", gen_device="cpu")
    T = wl.n_logical
    acc = binding.EmbeddingDwAccumulator(data.ids, 50, 64)
    half = layouts.chunked_packed(wl, sizes=[60, 40]).calls
    l0 = binding.Layout(half[0].row_logical, T)
    l1 = binding.Layout(half[1].row_logical, T)
    acc.contrib(data.dy[:60], l0)
    with pytest.raises(binding.RmsNormError) as ei:
        acc.contrib(data.dy[:60], l0)
    assert ei.value.code == binding.ECOVERAGE
    with pytest.raises(binding.RmsNormError) as ei:
        acc.finalize()
    assert ei.value.code == binding.ECOVERAGE
    acc.contrib(data.dy[60:], l1)
    d1 = acc.finalize().cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), acc.finalize().cpu().numpy().view(np.uint32))
    with pytest.raises(binding.RmsNormError) as ei:
        acc.contrib(data.dy[60:], l1)
    assert ei.value.code == binding.ESTATE
    acc.reset()
    acc.contrib(data.dy)
    assert np.array_equal(d1.view(np.uint32), acc.finalize().cpu().numpy().view(np.uint32))
    # a new batch's ids on the same accumulator
    ids2 = data.ids[::-1].copy()
    acc.set_ids(ids2)
    acc.contrib(data.dy)
    want = oracle.edo_v1_f32(ids2, inputs.bf16_bits(data.dy.cpu()), 50)
    assert np.array_equal(acc.finalize().cpu().numpy().view(np.uint32), want.view(np.uint32))
    with pytest.raises(binding.RmsNormError) as ei:
        acc.set_ids(np.full(T, 50, np.int32))              # id outside the vocabulary
    assert ei.value.code == binding.EINVAL
    acc.close()


@pytest.mark.parametrize("case", sorted(CASES))
def test_one_call_backward_is_the_accumulator_path(case):
    """det_embedding_bwd (single-block tokens folded straight into dE) gives
    the bits of contrib + finalize and of the EDO-v1 emulation."""
    dim, vocab, lengths, _ = CASES[case]
    wl = _wl(f"emb1_{case}", dim, vocab, lengths)
    data = adapters.make_embedding_inputs(wl, device="cuda", gen_device="cpu")
    counts = np.bincount(data.ids, minlength=vocab)
    print(f"[embedding] {case}: one-call backward, {int((counts > 0).sum())} tokens, "
          f"{int((counts > 64).sum())} with more than one block", flush=True)
    acc = binding.EmbeddingDwAccumulator(data.ids, vocab, dim)
    acc.contrib(data.dy)
    via_acc = acc.finalize().cpu().numpy()
    acc.reset()
    one = acc.backward(data.dy).cpu().numpy()
    assert np.array_equal(one.view(np.uint32), via_acc.view(np.uint32))
    want = oracle.edo_v1_f32(data.ids, inputs.bf16_bits(data.dy.cpu()), vocab)
    assert np.array_equal(one.view(np.uint32), want.view(np.uint32))
    # a dE buffer holding garbage is fully overwritten
    dE = torch.full((vocab, dim), float("nan"), device="cuda")
    acc.reset()
    acc.backward(data.dy, dE)
    assert np.array_equal(dE.cpu().numpy().view(np.uint32), want.view(np.uint32))
    acc.close()


def test_one_call_backward_protocol():
    wl = _wl("emb1_proto", 64, 50, [100])
    data = adapters.make_embedding_inputs(wl, device="cuda", gen_device="cpu")
    T = wl.n_logical
    acc = binding.EmbeddingDwAccumulator(data.ids, 50, 64)
    with pytest.raises(binding.RmsNormError) as ei:
        acc.backward(data.dy[:T - 1])                          # not every logical row
    assert ei.value.code == binding.ECOVERAGE
    half = layouts.chunked_packed(wl, sizes=[60, 40]).calls
    acc.contrib(data.dy[:60], binding.Layout(half[0].row_logical, T))
    with pytest.raises(binding.RmsNormError) as ei:
        acc.backward(data.dy)                                  # already holds a contribution
    assert ei.value.code == binding.ESTATE
    acc.reset()
    d1 = acc.backward(data.dy).cpu().numpy()
    with pytest.raises(binding.RmsNormError) as ei:
        acc.finalize()                                         # no partials are kept
    assert ei.value.code == binding.ESTATE
    with pytest.raises(binding.RmsNormError) as ei:
        acc.backward(data.dy)                                  # finalized
    assert ei.value.code == binding.ESTATE
    acc.reset()
    assert np.array_equal(d1.view(np.uint32), acc.backward(data.dy).cpu().numpy().view(np.uint32))
    # a new batch's ids
    ids2 = data.ids[::-1].copy()
    acc.set_ids(ids2)
    want = oracle.edo_v1_f32(ids2, inputs.bf16_bits(data.dy.cpu()), 50)
    assert np.array_equal(acc.backward(data.dy).cpu().numpy().view(np.uint32), want.view(np.uint32))
    acc.close()
