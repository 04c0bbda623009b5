"""C-ABI contract on the CPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from long_context_layers_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lightning_attn.h")

LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP = 0, 1, 2, 3
FAKE = 0x10000          # 16-byte aligned, never dereferenced by the checks below


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(binding.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.la_abi_version() == binding.ABI_VERSION


def test_status_strings(lib):
    for code in (LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP):
        s = lib.la_status_string(code).decode()
        assert s.startswith(["LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED", "LA_ERR_HIP"][code])
    assert lib.la_status_string(99).decode() == "unknown status"
    assert lib.la_status_string(-1).decode() == "unknown status"


PREFILL = ["la_prefill", "la_prefill_f32"]
DECODE = ["la_decode_step", "la_decode_step_f32"]


def _prefill_args(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000,
             out=FAKE + 0x400000, state=FAKE + 0x500000, B=1, H=2, N=0, d=64, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "slopes", "out", "state", "B", "H", "N", "d", "stream")]


def _decode_args(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000,
             state=FAKE + 0x400000, out=FAKE + 0x900000, B=1, H=2, d=64, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "slopes", "state", "out", "B", "H", "d", "stream")]


@pytest.mark.parametrize("fn", PREFILL)
def test_prefill_empty_sequence_is_a_noop(lib, fn):
    # N == 0 passes every check and returns before any HIP call; empty
    # activations may be null
    assert getattr(lib, fn)(*_prefill_args(N=0)) == LA_OK
    assert getattr(lib, fn)(*_prefill_args(N=0, q=None, k=None, v=None, out=None)) == LA_OK


@pytest.mark.parametrize("fn", PREFILL)
@pytest.mark.parametrize("bad,code", [
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(H=0), LA_ERR_INVALID_ARG),
    (dict(B=-1), LA_ERR_INVALID_ARG), (dict(N=-5), LA_ERR_INVALID_ARG),
    (dict(d=32), LA_ERR_UNSUPPORTED), (dict(d=96), LA_ERR_UNSUPPORTED),
    (dict(d=256), LA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 2), LA_ERR_INVALID_ARG),               # misaligned
    (dict(out=FAKE + 8), LA_ERR_INVALID_ARG),             # misaligned
])
def test_prefill_rejects_bad_arguments(lib, fn, bad, code):
    # N = 0 in every case: even a missing check could not reach a launch
    assert getattr(lib, fn)(*_prefill_args(**bad)) == code


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


# The cases below pass fake pointers with N >= 1 (or a decode step, which has
# no empty case): were a check missing, the call would reach a kernel launch,
# which must never happen with fake pointers on a machine that has a GPU.  So
# they run only where no GPU is visible; the GPU tests exercise the same rules
# with real tensors.
needs_no_gpu = pytest.mark.skipif(not _no_gpu(),
                                  reason="fake-pointer checks run only without a GPU")


@needs_no_gpu
@pytest.mark.parametrize("fn", PREFILL)
@pytest.mark.parametrize("bad", [
    dict(out=FAKE),                # out aliases q
    dict(out=FAKE + 0x100010),     # out overlaps k
    dict(out=FAKE + 0x500000),     # out aliases the state
    dict(B=2 ** 40, H=2 ** 40),    # size overflow
    dict(q=None), dict(k=None), dict(v=None), dict(out=None),   # null activations, N > 0
])
def test_prefill_rejects_aliasing_and_overflow(lib, fn, bad):
    assert getattr(lib, fn)(*_prefill_args(N=1, **bad)) == LA_ERR_INVALID_ARG


@needs_no_gpu
@pytest.mark.parametrize("fn", DECODE)
@pytest.mark.parametrize("bad,code", [
    (dict(q=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(out=None), LA_ERR_INVALID_ARG), (dict(slopes=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(H=-3), LA_ERR_INVALID_ARG),
    (dict(d=100), LA_ERR_UNSUPPORTED),
    (dict(state=FAKE + 0x400008), LA_ERR_INVALID_ARG),    # state not 16-byte aligned
    (dict(B=2 ** 40, H=2 ** 40), LA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(lib, fn, bad, code):
    assert getattr(lib, fn)(*_decode_args(**bad)) == code


@needs_no_gpu
@pytest.mark.parametrize("fn", DECODE)
def test_decode_rejects_aliasing(lib, fn):
    assert getattr(lib, fn)(*_decode_args(out=FAKE)) == LA_ERR_INVALID_ARG
    assert getattr(lib, fn)(*_decode_args(out=FAKE + 0x400000)) == LA_ERR_INVALID_ARG


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.prefill(x, x, x, torch.zeros(1), torch.zeros(1, 1, 64, 64))
    with pytest.raises(ValueError):
        binding.decode_step(x[:, :, 0], x[:, :, 0], x[:, :, 0], torch.zeros(1),
                            torch.zeros(1, 1, 64, 64))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(binding.LightningAttnError):
        # a fresh loader pointed at a path with no library
        saved = binding._lib
        binding._lib = None
        try:
            binding.load_library(str(tmp_path / "nope.so"))
        finally:
            binding._lib = saved


VARLEN = ["la_prefill_varlen", "la_prefill_varlen_f32"]


def _varlen_args(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000,
             cu=FAKE + 0x380000, nseq=3, out=FAKE + 0x400000, states=FAKE + 0x500000,
             H=2, T=0, d=64, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "slopes", "cu", "nseq", "out", "states", "H", "T", "d",
                           "stream")]


@pytest.mark.parametrize("fn", VARLEN)
def test_varlen_empty_batch_is_a_noop(lib, fn):
    # T == 0: every sequence is empty; returns before any HIP call (the
    # offsets are never read on the host)
    assert getattr(lib, fn)(*_varlen_args(T=0)) == LA_OK
    assert getattr(lib, fn)(*_varlen_args(T=0, q=None, k=None, v=None, out=None)) == LA_OK


@pytest.mark.parametrize("fn", VARLEN)
@pytest.mark.parametrize("bad,code", [
    (dict(cu=None), LA_ERR_INVALID_ARG), (dict(cu=FAKE + 4), LA_ERR_INVALID_ARG),
    (dict(nseq=0), LA_ERR_INVALID_ARG), (dict(nseq=-2), LA_ERR_INVALID_ARG),
    (dict(H=0), LA_ERR_INVALID_ARG), (dict(T=-1), LA_ERR_INVALID_ARG),
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(states=None), LA_ERR_INVALID_ARG),
    (dict(d=32), LA_ERR_UNSUPPORTED), (dict(d=256), LA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 2), LA_ERR_INVALID_ARG), (dict(states=FAKE + 8), LA_ERR_INVALID_ARG),
    (dict(nseq=2 ** 33, H=2 ** 31), LA_ERR_INVALID_ARG),     # state size overflows
    (dict(nseq=2 ** 26, H=64), LA_ERR_UNSUPPORTED),          # grid above 2^31 - 1
])
def test_varlen_rejects_bad_arguments(lib, fn, bad, code):
    # T = 0 in every case: even a missing check could not reach a launch
    assert getattr(lib, fn)(*_varlen_args(**bad)) == code


@needs_no_gpu
@pytest.mark.parametrize("fn", VARLEN)
@pytest.mark.parametrize("bad", [
    dict(out=FAKE),                # out aliases q
    dict(out=FAKE + 0x500000),     # out aliases the states
    dict(H=2 ** 62),               # size overflow (H * T * d)
    dict(q=None), dict(v=None), dict(out=None),   # null activations, T > 0
])
def test_varlen_rejects_aliasing_and_overflow(lib, fn, bad):
    assert getattr(lib, fn)(*_varlen_args(T=1, **bad)) == LA_ERR_INVALID_ARG


MULTI = ["la_decode_multi", "la_decode_multi_f32"]


def _multi_args(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000,
             n_commit=None, state=FAKE + 0x400000, out=FAKE + 0x900000, B=1, H=2, T=4, d=64,
             stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "slopes", "n_commit", "state", "out", "B", "H", "T",
                           "d", "stream")]


@needs_no_gpu
@pytest.mark.parametrize("fn", MULTI)
@pytest.mark.parametrize("bad,code", [
    (dict(T=0), LA_ERR_INVALID_ARG), (dict(T=-1), LA_ERR_INVALID_ARG),
    (dict(T=9), LA_ERR_UNSUPPORTED), (dict(T=64), LA_ERR_UNSUPPORTED),
    (dict(n_commit=FAKE + 0xa00002), LA_ERR_INVALID_ARG),     # misaligned int32 pointer
    (dict(q=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(out=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(H=0), LA_ERR_INVALID_ARG),
    (dict(d=96), LA_ERR_UNSUPPORTED),
    (dict(out=FAKE), LA_ERR_INVALID_ARG),                     # out aliases q
    (dict(out=FAKE + 0x400000), LA_ERR_INVALID_ARG),          # out aliases the state
    (dict(state=FAKE + 0x400008), LA_ERR_INVALID_ARG),        # misaligned state
    (dict(B=2 ** 40, H=2 ** 40), LA_ERR_INVALID_ARG),         # size overflow
])
def test_decode_multi_rejects_bad_arguments(lib, fn, bad, code):
    # every case fails a host check (a missing one would launch on fake
    # pointers, hence no-GPU machines only)
    assert getattr(lib, fn)(*_multi_args(**bad)) == code


def _rope_args(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, stride=3 * 2 * 64, qw=FAKE + 0x300000,
             kw=FAKE + 0x310000, theta=6e6, rot=64, pos0=0, eps=1e-6, qo=FAKE + 0x400000,
             ko=FAKE + 0x500000, vo=FAKE + 0x600000, B=1, N=0, H=2, d=64, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "stride", "qw", "kw", "theta", "rot", "pos0", "eps",
                           "qo", "ko", "vo", "B", "N", "H", "d", "stream")]


def _gate_args(**kw):
    a = dict(o=FAKE, ob=2 * 3 * 64, oh=3 * 64, ot=64, g=FAKE + 0x100000, gstride=2 * 64,
             w=FAKE + 0x300000, group=64, eps=1e-6, y=FAKE + 0x400000, B=1, N=0, H=2, d=64,
             stream=None)
    a.update(kw)
    return [a[n] for n in ("o", "ob", "oh", "ot", "g", "gstride", "w", "group", "eps", "y", "B",
                           "N", "H", "d", "stream")]


def test_layer_ops_empty_is_a_noop(lib):
    assert lib.la_qk_norm_rope(*_rope_args(N=0)) == LA_OK
    assert lib.la_qk_norm_rope(*_rope_args(N=0, q=None, k=None, v=None, qo=None, ko=None,
                                           vo=None)) == LA_OK
    assert lib.la_group_norm_gate(*_gate_args(N=0)) == LA_OK
    assert lib.la_group_norm_gate(*_gate_args(N=0, o=None, g=None, y=None)) == LA_OK


@pytest.mark.parametrize("bad,code", [
    (dict(rot=48), LA_ERR_UNSUPPORTED), (dict(rot=8), LA_ERR_UNSUPPORTED),
    (dict(rot=128), LA_ERR_UNSUPPORTED),                    # > d
    (dict(theta=1.0), LA_ERR_INVALID_ARG), (dict(theta=float("nan")), LA_ERR_INVALID_ARG),
    (dict(pos0=-1), LA_ERR_INVALID_ARG), (dict(eps=-1.0), LA_ERR_INVALID_ARG),
    (dict(stride=100), LA_ERR_INVALID_ARG),                 # < H*d
    (dict(stride=3 * 2 * 64 + 4), LA_ERR_INVALID_ARG),      # not a multiple of 8
    (dict(qw=None), LA_ERR_INVALID_ARG), (dict(kw=FAKE + 0x310004), LA_ERR_INVALID_ARG),
    (dict(d=96), LA_ERR_UNSUPPORTED), (dict(B=0), LA_ERR_INVALID_ARG),
    (dict(H=0), LA_ERR_INVALID_ARG), (dict(N=-1), LA_ERR_INVALID_ARG),
])
def test_qk_norm_rope_rejects_bad_arguments(lib, bad, code):
    # N = 0 unless the case sets it: a missing check could not reach a launch
    assert lib.la_qk_norm_rope(*_rope_args(**bad)) == code


@pytest.mark.parametrize("bad,code", [
    (dict(group=4), LA_ERR_UNSUPPORTED), (dict(group=48), LA_ERR_UNSUPPORTED),
    (dict(group=128), LA_ERR_UNSUPPORTED),                  # > d
    (dict(gstride=64), LA_ERR_INVALID_ARG), (dict(eps=float("nan")), LA_ERR_INVALID_ARG),
    (dict(w=None), LA_ERR_INVALID_ARG), (dict(w=FAKE + 0x300008), LA_ERR_INVALID_ARG),
    (dict(d=32), LA_ERR_UNSUPPORTED), (dict(B=-1), LA_ERR_INVALID_ARG),
    (dict(ot=68), LA_ERR_INVALID_ARG), (dict(oh=-64), LA_ERR_INVALID_ARG),   # o strides
])
def test_group_norm_gate_rejects_bad_arguments(lib, bad, code):
    assert lib.la_group_norm_gate(*_gate_args(**bad)) == code


@needs_no_gpu
@pytest.mark.parametrize("bad", [dict(qo=FAKE), dict(vo=FAKE + 0x100000), dict(ko=FAKE + 0x400000),
                                 dict(q=None), dict(vo=None), dict(v=None), dict(q=FAKE + 8),
                                 # in place: q and k rows interleaved in one buffer must not share elements
                                 dict(k=FAKE + 64, qo=FAKE, ko=FAKE + 64, v=None, vo=None),
                                 dict(k=FAKE + 3 * 2 * 64 * 2 - 128, qo=FAKE,
                                      ko=FAKE + 3 * 2 * 64 * 2 - 128, v=None, vo=None),
                                 # in place with v rows overlapping q's
                                 dict(v=FAKE + 128, qo=FAKE, ko=FAKE + 0x100000),
                                 # only q in place
                                 dict(qo=FAKE, v=None, vo=None)])
def test_qk_norm_rope_rejects_overlap_and_nulls(lib, bad):
    assert lib.la_qk_norm_rope(*_rope_args(N=3, **bad)) == LA_ERR_INVALID_ARG


@needs_no_gpu
@pytest.mark.parametrize("bad", [dict(y=FAKE), dict(y=FAKE + 0x100000), dict(o=None), dict(g=FAKE + 2),
                                 dict(y=FAKE + 2 * 3 * 64 * 2 - 16)])   # y inside a strided o's span
def test_group_norm_gate_rejects_overlap_and_nulls(lib, bad):
    assert lib.la_group_norm_gate(*_gate_args(N=3, **bad)) == LA_ERR_INVALID_ARG


STRIDED = ["la_prefill_strided", "la_prefill_varlen_strided"]
# the argument checks are shared by the zero-start packed call (which, unlike
# the others, launches even with no tokens: it writes the empty sequences' states)
STRIDED_CHECKS = STRIDED + ["la_prefill_varlen_from_zero"]


def _strided_args(fn, **kw):
    # defaults: B=1, H=2, N (or T) tokens, d=64, token-major [B,N,H,d] layouts
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000,
             cu=FAKE + 0x380000, nseq=3, out=FAKE + 0x400000, state=FAKE + 0x500000,
             B=1, H=2, N=0, d=64, ib=None, ih=64, it=128, ob=None, oh=64, ot=128, stream=None)
    a.update(kw)
    if fn == "la_prefill_strided":
        ib = a["ib"] if a["ib"] is not None else a["N"] * a["it"]
        ob = a["ob"] if a["ob"] is not None else a["N"] * a["ot"]
        return [a[n] for n in ("q", "k", "v", "slopes", "out", "state", "B", "H", "N", "d")] + \
            [ib, a["ih"], a["it"], ob, a["oh"], a["ot"], a["stream"]]
    return [a[n] for n in ("q", "k", "v", "slopes", "cu", "nseq", "out", "state", "H", "N", "d",
                           "ih", "it", "oh", "ot", "stream")]


@pytest.mark.parametrize("fn", STRIDED)
def test_strided_empty_is_a_noop(lib, fn):
    assert getattr(lib, fn)(*_strided_args(fn, N=0)) == LA_OK
    assert getattr(lib, fn)(*_strided_args(fn, N=0, q=None, k=None, v=None, out=None)) == LA_OK


@pytest.mark.parametrize("fn", STRIDED_CHECKS)
@pytest.mark.parametrize("bad,code", [
    (dict(ih=60), LA_ERR_INVALID_ARG), (dict(it=-128), LA_ERR_INVALID_ARG),   # not a multiple of 8 / < 0
    (dict(oh=4), LA_ERR_INVALID_ARG),
    (dict(oh=32), LA_ERR_INVALID_ARG),              # output heads share elements
    (dict(it=32), LA_ERR_INVALID_ARG), (dict(ot=0), LA_ERR_INVALID_ARG),   # token stride < d
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(d=32), LA_ERR_UNSUPPORTED), (dict(q=FAKE + 8), LA_ERR_INVALID_ARG),
    (dict(out=FAKE + 0x400008), LA_ERR_INVALID_ARG),
])
def test_strided_rejects_bad_arguments(lib, fn, bad, code):
    # no tokens: even a missing check could not reach a launch
    if fn == "la_prefill_varlen_from_zero" and bad == dict(state=None):
        code = LA_OK          # from zero the states may be null: outputs only
    assert getattr(lib, fn)(*_strided_args(fn, N=0, **bad)) == code


@needs_no_gpu
@pytest.mark.parametrize("fn", STRIDED_CHECKS)
@pytest.mark.parametrize("bad,code", [
    (dict(ot=64), LA_ERR_INVALID_ARG),              # output tokens overlap heads (ot < H*d)
    (dict(ot=0), LA_ERR_INVALID_ARG),               # every output token on one row
    (dict(out=FAKE + 0x200000 + 256), LA_ERR_INVALID_ARG),   # out inside v's span
    (dict(out=FAKE + 0x500000), LA_ERR_INVALID_ARG),         # out aliases the state
    (dict(it=2 ** 24 + 8), LA_ERR_UNSUPPORTED), (dict(ot=2 ** 24 + 8), LA_ERR_UNSUPPORTED),
    (dict(q=None), LA_ERR_INVALID_ARG), (dict(out=None), LA_ERR_INVALID_ARG),
    (dict(it=2 ** 62, ib=0), LA_ERR_INVALID_ARG),    # span overflows
])
def test_strided_rejects_overlap_and_limits(lib, fn, bad, code):
    assert getattr(lib, fn)(*_strided_args(fn, N=3, **bad)) == code


def _fold_args(lens=(3, 4, 5), **kw):
    arr = (ctypes.c_int64 * len(lens))(*lens)
    a = dict(loc=FAKE, lensp=ctypes.cast(arr, ctypes.c_void_p).value, nshards=len(lens), rank=2,
             slopes=FAKE + 0x900000, init=FAKE + 0xa00000, out=FAKE + 0xb00000, B=1, H=2, d=64,
             stream=None)
    a.update(kw)
    return arr, [a[n] for n in ("loc", "lensp", "nshards", "rank", "slopes", "init", "out", "B",
                                "H", "d", "stream")]


@needs_no_gpu
@pytest.mark.parametrize("bad,code", [
    (dict(nshards=0, rank=0), LA_ERR_INVALID_ARG), (dict(rank=-1), LA_ERR_INVALID_ARG),
    (dict(rank=4), LA_ERR_INVALID_ARG),                        # rank > nshards
    (dict(nshards=65, rank=1), LA_ERR_UNSUPPORTED),
    (dict(lensp=None), LA_ERR_INVALID_ARG), (dict(loc=None), LA_ERR_INVALID_ARG),
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(out=None), LA_ERR_INVALID_ARG),
    (dict(d=96), LA_ERR_UNSUPPORTED), (dict(B=0), LA_ERR_INVALID_ARG),
    (dict(out=FAKE + 0xb00008), LA_ERR_INVALID_ARG),           # misaligned
    (dict(out=FAKE + 0x4000), LA_ERR_INVALID_ARG),             # inside the local states
    (dict(out=FAKE + 0xa00010), LA_ERR_INVALID_ARG),           # partly over state_init
])
def test_cp_fold_rejects_bad_arguments(lib, bad, code):
    arr, args = _fold_args(**bad)
    assert lib.la_cp_fold(*args) == code


@needs_no_gpu
@pytest.mark.parametrize("lens,code", [((3, -1, 5), LA_ERR_INVALID_ARG),
                                       ((3, 2 ** 31, 5), LA_ERR_UNSUPPORTED)])
def test_cp_fold_rejects_bad_lengths(lib, lens, code):
    arr, args = _fold_args(lens=lens)
    assert lib.la_cp_fold(*args) == code


def _correct_args(**kw):
    a = dict(q=FAKE, slopes=FAKE + 0x100000, state=FAKE + 0x200000, out=FAKE + 0x300000, B=1,
             H=2, L=0, d=64, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "slopes", "state", "out", "B", "H", "L", "d", "stream")]


def test_cp_correct_empty_shard_is_a_noop(lib):
    assert lib.la_cp_correct(*_correct_args(L=0)) == LA_OK
    assert lib.la_cp_correct(*_correct_args(L=0, q=None, out=None)) == LA_OK


@pytest.mark.parametrize("bad,code", [
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(L=-1), LA_ERR_INVALID_ARG),
    (dict(d=32), LA_ERR_UNSUPPORTED), (dict(q=FAKE + 8), LA_ERR_INVALID_ARG),
    (dict(state=FAKE + 0x200004), LA_ERR_INVALID_ARG),
])
def test_cp_correct_rejects_bad_arguments(lib, bad, code):
    assert lib.la_cp_correct(*_correct_args(**bad)) == code


@needs_no_gpu
@pytest.mark.parametrize("bad,code", [
    (dict(out=FAKE), LA_ERR_INVALID_ARG),                      # out aliases q
    (dict(out=FAKE + 0x200000), LA_ERR_INVALID_ARG),           # out aliases the state
    (dict(q=None), LA_ERR_INVALID_ARG), (dict(out=None), LA_ERR_INVALID_ARG),
    (dict(L=2 ** 31 - 1, out=FAKE + 2 ** 45), LA_ERR_UNSUPPORTED),
])
def test_cp_correct_rejects_overlap_and_limits(lib, bad, code):
    assert lib.la_cp_correct(*_correct_args(L=bad.pop("L", 5), **bad)) == code


def test_peak_probe_library_loads_and_rejects_bad_arguments():
    # the benchmark's ceiling probes (lib/liblapeak.so): every call checks its
    # arguments on the host before any launch
    from long_context_layers_amd import build
    peak = ctypes.CDLL(build.PEAK_LIB)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    for name in ("la_peak_mfma_bf16", "la_peak_read", "la_peak_write", "la_peak_copy",
                 "la_peak_update", "la_peak_mix3", "la_peak_mfma_chains",
                 "la_peak_stream_persistent", "la_peak_pair_pattern"):
        assert hasattr(peak, name), name
    peak.la_peak_mfma_bf16.argtypes = [I64, I64, P, P]
    peak.la_peak_read.argtypes = [P, I64, P, P]
    peak.la_peak_write.argtypes = [P, I64, P]
    peak.la_peak_copy.argtypes = [P, P, I64, P]
    assert peak.la_peak_mfma_chains() == 4
    assert peak.la_peak_mfma_bf16(0, 1, FAKE, None) == -1
    assert peak.la_peak_mfma_bf16(1, 0, FAKE, None) == -1
    assert peak.la_peak_mfma_bf16(1, 1, None, None) == -1
    assert peak.la_peak_read(FAKE, 24, FAKE, None) == -1          # not a multiple of 16
    assert peak.la_peak_read(None, 32, FAKE, None) == -1
    assert peak.la_peak_write(FAKE, 0, None) == -1
    assert peak.la_peak_copy(FAKE, None, 32, None) == -1
    peak.la_peak_update.argtypes = [P, I64, P]
    assert peak.la_peak_update(FAKE, 8, None) == -1
    peak.la_peak_mix3.argtypes = [P, P, P, P, I64, P]
    assert peak.la_peak_mix3(FAKE, FAKE, FAKE, None, 65536, None) == -1
    assert peak.la_peak_mix3(FAKE, FAKE, FAKE, FAKE, 65536 + 16, None) == -1    # not whole chunks
    f = peak.la_peak_stream_persistent
    f.argtypes = [ctypes.c_int, P, P, P, P, I64, I64, P, P]
    burst = 256 * 32 * 16                                   # 128 KB per workgroup burst
    assert f(0, FAKE, None, None, None, 4 * burst, 4, None, None) == -1        # read needs a sink
    assert f(1, None, None, None, None, 4 * burst, 4, None, None) == -1        # write needs d
    assert f(2, FAKE, FAKE, None, FAKE, 4 * burst, 4, None, None) == -1        # mix3 needs a, b, c, d
    assert f(2, FAKE, FAKE, FAKE, FAKE, 4 * burst + 16, 4, None, None) == -1   # not whole bursts
    assert f(2, FAKE, FAKE, FAKE, FAKE, 4 * burst, 0, None, None) == -1        # no workgroups
    assert f(2, FAKE, FAKE, FAKE, FAKE, 4 * burst, 65537, None, None) == -1    # too many
    assert f(3, FAKE, FAKE, FAKE, FAKE, 4 * burst, 4, FAKE, None) == -1        # unknown kind
    pp = peak.la_peak_pair_pattern
    pp.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P, P, I64, I64, P]
    assert pp(0, 1, FAKE, FAKE, FAKE, None, 8, 64, None) == -1      # null output
    assert pp(0, 1, FAKE, FAKE, FAKE, FAKE, 12, 64, None) == -1     # slots not a multiple of 8
    assert pp(1, 1, FAKE, FAKE, FAKE, FAKE, 8, 100, None) == -1     # tokens not whole blocks
    assert pp(1, 4, FAKE, FAKE, FAKE, FAKE, 8, 128, None) == -1     # not whole groups of 4 blocks
    assert pp(2, 1, FAKE, FAKE, FAKE, FAKE, 0, 64, None) == -1      # no slots
    assert pp(3, 1, FAKE, FAKE, FAKE, FAKE, 8, 64, None) == -1      # unknown mode
    assert pp(0, 2, FAKE, FAKE, FAKE, FAKE, 8, 256, None) == -1     # 1 or 4 blocks in flight


def _dstr_args(**kw):
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000, nc=None,
             state=FAKE + 0x400000, out=FAKE + 0x900000, B=2, H=2, T=3, d=64, sb=3 * 2 * 64,
             sh=64, st=6 * 64 * 3, stream=None)
    a.update(kw)
    return a


@needs_no_gpu
@pytest.mark.parametrize("bad,code", [
    (dict(q=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(d=96), LA_ERR_UNSUPPORTED), (dict(B=0), LA_ERR_INVALID_ARG),
    (dict(sb=-8), LA_ERR_INVALID_ARG),                          # negative stride
    (dict(q=FAKE + 1), LA_ERR_INVALID_ARG),                     # not 2-byte aligned
    (dict(state=FAKE + 0x400008), LA_ERR_INVALID_ARG),
    (dict(out=FAKE + 64), LA_ERR_INVALID_ARG),                  # out inside q's span
    (dict(out=FAKE + 0x400000), LA_ERR_INVALID_ARG),            # out over the state
])
def test_decode_step_strided_rejects_bad_arguments(lib, bad, code):
    a = _dstr_args(**bad)
    assert lib.la_decode_step_strided(a["q"], a["k"], a["v"], a["slopes"], a["state"], a["out"],
                                      a["B"], a["H"], a["d"], a["sb"], a["sh"], a["stream"]) == code


@needs_no_gpu
@pytest.mark.parametrize("bad,code", [
    (dict(T=0), LA_ERR_INVALID_ARG), (dict(T=9), LA_ERR_UNSUPPORTED),
    (dict(nc=FAKE + 0xa00002), LA_ERR_INVALID_ARG),             # misaligned n_commit
    (dict(v=None), LA_ERR_INVALID_ARG), (dict(st=-64), LA_ERR_INVALID_ARG),
    (dict(out=FAKE + 0x200010), LA_ERR_INVALID_ARG),            # out inside v's span
])
def test_decode_multi_strided_rejects_bad_arguments(lib, bad, code):
    a = _dstr_args(**bad)
    assert lib.la_decode_multi_strided(a["q"], a["k"], a["v"], a["slopes"], a["nc"], a["state"],
                                       a["out"], a["B"], a["H"], a["T"], a["d"], a["sb"], a["sh"],
                                       a["st"], a["stream"]) == code


@pytest.mark.parametrize("nseq,H,T,d,walks_null,code", [
    (0, 64, 10, 128, False, LA_ERR_INVALID_ARG),
    (2, 0, 10, 128, False, LA_ERR_INVALID_ARG),
    (2, 64, -1, 128, False, LA_ERR_INVALID_ARG),
    (2, 64, 10, 128, True, LA_ERR_INVALID_ARG),
    (2, 64, 10, 96, False, LA_ERR_UNSUPPORTED),
    (2, 64, 10, 32, False, LA_ERR_UNSUPPORTED),
])
def test_varlen_plan_rejects_bad_arguments(lib, nseq, H, T, d, walks_null, code):
    walks = ctypes.c_int(7)
    arg = None if walks_null else ctypes.byref(walks)
    assert lib.la_prefill_varlen_plan(nseq, H, T, d, arg) == code
    assert walks.value == 7            # untouched on error


def _prefill_ws_args(workspace=None, ws_bytes=0, **kw):
    a = _prefill_args(**kw)
    return a[:-1] + [workspace, ws_bytes, a[-1]]


@pytest.mark.parametrize("bad,code", [
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(H=0), LA_ERR_INVALID_ARG),
    (dict(N=-5), LA_ERR_INVALID_ARG), (dict(d=96), LA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 2), LA_ERR_INVALID_ARG), (dict(out=FAKE + 8), LA_ERR_INVALID_ARG),
])
def test_prefill_ws_rejects_bad_arguments(lib, bad, code):
    # the workspace prefill takes la_prefill's checks first (N = 0: no launch)
    assert lib.la_prefill_ws(*_prefill_ws_args(**bad)) == code
    assert lib.la_prefill_ws(*_prefill_ws_args(N=0)) == LA_OK


@pytest.mark.parametrize("B,H,N,d,null,code", [
    (1, 32, 262144, 128, True, LA_ERR_INVALID_ARG), (0, 32, 1024, 128, False, LA_ERR_INVALID_ARG),
    (1, 0, 1024, 128, False, LA_ERR_INVALID_ARG), (1, 32, -1, 128, False, LA_ERR_INVALID_ARG),
    (1, 32, 1024, 96, False, LA_ERR_UNSUPPORTED),
])
def test_prefill_workspace_bytes_rejects_bad_arguments(lib, B, H, N, d, null, code):
    n = ctypes.c_int64(-1)
    assert lib.la_prefill_workspace_bytes(B, H, N, d, None if null else ctypes.byref(n)) == code


@needs_no_gpu
def test_prefill_workspace_bytes_without_a_device_is_zero(lib):
    # no device: no compute units to fill, so no split and no workspace
    for B, H, N in ((1, 32, 262144), (1, 1, 1 << 20), (4, 64, 4096)):
        n = ctypes.c_int64(-1)
        assert lib.la_prefill_workspace_bytes(B, H, N, 128, ctypes.byref(n)) == LA_OK
        assert n.value == 0


@pytest.mark.parametrize("bad,code", [
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(H=0), LA_ERR_INVALID_ARG),
    (dict(N=-5), LA_ERR_INVALID_ARG), (dict(d=96), LA_ERR_UNSUPPORTED),
    (dict(q=FAKE + 8), LA_ERR_INVALID_ARG), (dict(out=FAKE + 8), LA_ERR_INVALID_ARG),
])
def test_prefill_f32_ws_rejects_bad_arguments(lib, bad, code):
    # the fp32 workspace prefill takes la_prefill_f32's checks first (16-byte
    # aligned fp32 tensors; N = 0: no launch)
    assert lib.la_prefill_f32_ws(*_prefill_ws_args(**bad)) == code
    assert lib.la_prefill_f32_ws(*_prefill_ws_args(N=0)) == LA_OK


@pytest.mark.parametrize("B,H,N,d,null,code", [
    (1, 64, 32768, 128, True, LA_ERR_INVALID_ARG), (0, 32, 1024, 128, False, LA_ERR_INVALID_ARG),
    (1, 0, 1024, 128, False, LA_ERR_INVALID_ARG), (1, 32, -1, 128, False, LA_ERR_INVALID_ARG),
    (1, 32, 1024, 96, False, LA_ERR_UNSUPPORTED),
])
def test_prefill_f32_workspace_bytes_rejects_bad_arguments(lib, B, H, N, d, null, code):
    n = ctypes.c_int64(-1)
    assert lib.la_prefill_f32_workspace_bytes(B, H, N, d, None if null else ctypes.byref(n)) == code


@needs_no_gpu
def test_prefill_f32_workspace_bytes_without_a_device_is_zero(lib):
    for B, H, N in ((1, 64, 32768), (1, 1, 1 << 20), (4, 64, 4096)):
        n = ctypes.c_int64(-1)
        assert lib.la_prefill_f32_workspace_bytes(B, H, N, 128, ctypes.byref(n)) == LA_OK
        assert n.value == 0


@pytest.mark.parametrize("bad,code", [
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(N=-5), LA_ERR_INVALID_ARG),
    (dict(d=96), LA_ERR_UNSUPPORTED), (dict(q=FAKE + 2), LA_ERR_INVALID_ARG),
])
def test_prefill_noalloc_rejects_bad_arguments(lib, bad, code):
    # the allocation-free prefill takes la_prefill's checks first (N = 0: no launch)
    assert lib.la_prefill_noalloc(*_prefill_args(**bad)) == code
    assert lib.la_prefill_noalloc(*_prefill_args(N=0)) == LA_OK


def _fused_args(**kw):
    # la_prefill_qk_norm_rope_ws; defaults: B=1, H=2, no tokens, d=128,
    # token-major [B,N,3*H*d] projection rows, the layer's prologue constants
    a = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, slopes=FAKE + 0x300000,
             qw=FAKE + 0x340000, kw=FAKE + 0x360000, theta=6e6, rot=64, pos0=0, eps=1e-6,
             out=FAKE + 0x400000, state=FAKE + 0x500000, B=1, H=2, N=0, d=128,
             ib=0, ih=128, it=768, ob=0, oh=128, ot=256, ws=None, wsb=0, stream=None)
    a.update(kw)
    return [a[n] for n in ("q", "k", "v", "slopes", "qw", "kw", "theta", "rot", "pos0", "eps",
                           "out", "state", "B", "H", "N", "d", "ib", "ih", "it", "ob", "oh", "ot",
                           "ws", "wsb", "stream")]


def test_fused_prologue_prefill_empty_is_a_noop(lib):
    assert lib.la_prefill_qk_norm_rope_ws(*_fused_args()) == LA_OK
    assert lib.la_prefill_qk_norm_rope_ws(*_fused_args(q=None, k=None, v=None, out=None)) == LA_OK
    for rot in (0, 16, 32, 128):
        assert lib.la_prefill_qk_norm_rope_ws(*_fused_args(rot=rot)) == LA_OK


@pytest.mark.parametrize("bad,code", [
    (dict(d=64), LA_ERR_UNSUPPORTED), (dict(d=96), LA_ERR_UNSUPPORTED),
    (dict(rot=48), LA_ERR_UNSUPPORTED), (dict(rot=256), LA_ERR_UNSUPPORTED),
    (dict(rot=8), LA_ERR_UNSUPPORTED),
    (dict(qw=None), LA_ERR_INVALID_ARG), (dict(kw=None), LA_ERR_INVALID_ARG),
    (dict(kw=FAKE + 0x360004), LA_ERR_INVALID_ARG),             # weights not 16-byte aligned
    (dict(theta=1.0), LA_ERR_INVALID_ARG), (dict(theta=float("nan")), LA_ERR_INVALID_ARG),
    (dict(eps=0.0), LA_ERR_INVALID_ARG), (dict(eps=1e-40), LA_ERR_INVALID_ARG),   # subnormal
    (dict(eps=float("inf")), LA_ERR_INVALID_ARG), (dict(eps=float("nan")), LA_ERR_INVALID_ARG),
    (dict(eps=-1e-6), LA_ERR_INVALID_ARG),
    (dict(pos0=-1), LA_ERR_INVALID_ARG), (dict(pos0=2 ** 63 - 1, N=1), LA_ERR_INVALID_ARG),
    (dict(slopes=None), LA_ERR_INVALID_ARG), (dict(state=None), LA_ERR_INVALID_ARG),
    (dict(ih=60), LA_ERR_INVALID_ARG), (dict(it=64), LA_ERR_INVALID_ARG),   # stride rules
    (dict(B=0), LA_ERR_INVALID_ARG), (dict(N=-1), LA_ERR_INVALID_ARG),
])
def test_fused_prologue_prefill_rejects_bad_arguments(lib, bad, code):
    # no tokens (or a rejected position range): no check can reach a launch
    assert lib.la_prefill_qk_norm_rope_ws(*_fused_args(**bad)) == code


@needs_no_gpu
@pytest.mark.parametrize("bad,code", [
    (dict(cu=None), LA_ERR_INVALID_ARG), (dict(cu=FAKE + 0x380004), LA_ERR_INVALID_ARG),
    (dict(nseq=0), LA_ERR_INVALID_ARG), (dict(H=0), LA_ERR_INVALID_ARG),
    (dict(N=-1), LA_ERR_INVALID_ARG), (dict(state=None, N=-1), LA_ERR_INVALID_ARG),
    (dict(state=None, slopes=None), LA_ERR_INVALID_ARG), (dict(state=None, d=32), LA_ERR_UNSUPPORTED),
])
def test_varlen_from_zero_rejects_bad_arguments(lib, bad, code):
    assert lib.la_prefill_varlen_from_zero(*_strided_args("la_prefill_varlen_from_zero", **bad)) == code


@needs_no_gpu
def test_varlen_from_zero_without_states_and_tokens_is_a_noop(lib):
    # null states: outputs only; with no tokens there is nothing to write (the
    # same call with states writes the empty sequences' zero states)
    assert lib.la_prefill_varlen_from_zero(*_strided_args("la_prefill_varlen_from_zero", N=0,
                                                          state=None)) == LA_OK
