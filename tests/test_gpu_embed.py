"""Bit-exact parity of the Q4 embedding lookups with the oracle, on the packed
table (q4_0_embed) and on the same table as GGUF blocks (q4_0_embed_gguf):
rows of the dequantized table in the requested order, duplicates repeated,
NaN rows for ids outside the table; small ragged tables, rows longer than
the GGUF lookup's 256-block run, the full 131072 x 3072 table (the LM head's)
with a prefill-sized batch of ids, and agreement with q4_0_dequant of the
whole table."""

import numpy as np
import pytest
import torch

from oracle import q4_0_oracle as O
import q4_weight_only_amd as q4
from q4_weight_only_amd import inputs

from gpu_helpers import DEV, device_weight_from_f32, say

pytestmark = pytest.mark.gpu

SHAPES = [(16, 32), (40, 96), (200, 384), (1040, 1280), (33, 3072), (24, 9376)]
FORMS = ["packed", "gguf"]


def _lookup(form, pw, blocks, ids_dev):
    if form == "packed":
        return q4.embed(pw, ids_dev)
    return q4.embed_gguf(blocks, pw.n, pw.k, ids_dev)


def _ids(n, count, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, n, count).astype(np.int32)
    return np.concatenate([[0, n - 1], ids, ids[:3], [-1, n, np.iinfo(np.int32).max, np.iinfo(np.int32).min]]).astype(np.int32)


def _same(got, want):
    """Bitwise equal, with every NaN row NaN in both."""
    assert got.shape == want.shape
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("n,k", SHAPES)
def test_embed_parity(n, k, form):
    w = inputs.weights_f32((n, k), seed=41, tags=(n, k))
    pw, blocks = device_weight_from_f32(w)
    gb = blocks.cpu().numpy()
    assert np.array_equal(gb, O.quantize(w))
    ids = _ids(n, 3 * n, 41)
    say("embed", form, n, k, len(ids))
    got = _lookup(form, pw, blocks, torch.from_numpy(ids).to(DEV)).cpu().numpy()
    _same(got, O.embed(gb, n, k, ids))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("n,k", [(40, 96), (1040, 1280)])
def test_embed_all_rows_equals_dequant(n, k, form):
    w = inputs.weights_f32((n, k), seed=42, tags=(n, k))
    pw, blocks = device_weight_from_f32(w)
    say("embed vs dequant", form, n, k)
    got = _lookup(form, pw, blocks, torch.arange(n, dtype=torch.int32, device=DEV)).cpu().numpy()
    full = q4.dequant(pw).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), full.view(np.uint32))


@pytest.mark.parametrize("form", FORMS)
def test_embed_empty(form):
    w = inputs.weights_f32((16, 64), seed=43, tags=(1,))
    pw, blocks = device_weight_from_f32(w)
    out = _lookup(form, pw, blocks, torch.empty(0, dtype=torch.int32, device=DEV))
    assert tuple(out.shape) == (0, 64)


def test_embed_forms_agree_with_non_finite_scales():
    """Scales of +-inf and NaN: both lookups give the same bits as the oracle."""
    n, k = 48, 320
    gb = O.quantize(inputs.weights_f32((n, k), seed=45)).copy()
    d_bits = gb[:, :, :2].view(np.uint16)
    d_bits[3, 1, 0] = 0x7C00
    d_bits[5, 9, 0] = 0xFC00
    d_bits[7, 0, 0] = 0x7E00
    blocks = torch.from_numpy(gb).to(DEV)
    pw = q4.pack(blocks, n, k)
    ids = torch.from_numpy(np.array([3, 5, 7, 0, 3], dtype=np.int32)).to(DEV)
    say("embed non-finite scales")
    a = q4.embed(pw, ids).cpu().numpy()
    b = q4.embed_gguf(blocks, n, k, ids).cpu().numpy()
    with np.errstate(invalid="ignore"):
        want = O.embed(gb, n, k, ids.cpu().numpy())
    _same(a, want)
    _same(b, want)


def test_embed_full_table_prefill_batch():
    """The 131072 x 3072 table (the LM head's weights) and 2048 ids."""
    spec = inputs.workload(3)[1][0][0]
    w = spec.weight(0)
    n, k = w.shape
    pw, blocks = device_weight_from_f32(w)
    ids = _ids(n, 2048, 44)
    say("embed full table", n, k, len(ids))
    ids_dev = torch.from_numpy(ids).to(DEV)
    got = q4.embed(pw, ids_dev).cpu().numpy()
    got_gguf = q4.embed_gguf(blocks, n, k, ids_dev).cpu().numpy()
    valid = ids[(ids >= 0) & (ids < n)]
    uniq, inv = np.unique(valid, return_inverse=True)
    rows = blocks.view(n, -1)[torch.from_numpy(uniq.astype(np.int64)).to(DEV)].cpu().numpy()
    assert np.array_equal(rows, O.quantize(w[uniq]).reshape(len(uniq), -1))
    want = np.full((len(ids), k), np.nan, dtype=np.float32)
    want[(ids >= 0) & (ids < n)] = O.embed(rows, len(uniq), k, inv)
    _same(got, want)
    _same(got_gguf, want)
