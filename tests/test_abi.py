"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, sizes workspaces, and rejects invalid host-checkable
arguments before touching the device (no compute calls here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")
LIB = os.path.join(ROOT, "semi_ar_draft_round_amd", "libdspark.so")

EINVAL, EDTYPE, EWORKSPACE = 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from semi_ar_draft_round_amd import build
        build.build()
    from semi_ar_draft_round_amd import binding
    return binding.load_library(LIB)


def test_header_declares_the_four_calls():
    fns = declared_functions()
    for name in ("dspark_markov_sample", "dspark_confidence", "dspark_schedule", "dspark_verify",
                 "dspark_workspace_size", "dspark_status_string"):
        assert name in fns


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    from semi_ar_draft_round_amd import binding
    assert sorted(binding.EXPORTED) == declared_functions()


def test_status_strings(lib):
    for s in range(7):
        assert b"unknown" not in lib.dspark_status_string(s)
    assert b"unknown" in lib.dspark_status_string(99)


def test_workspace_sizes(lib):
    from semi_ar_draft_round_amd import binding as B
    n_c = (129280 + 63) // 64
    ws = B.dspark_workspace_size(B.WS_SAMPLE, 128, 16, 129280, 256)
    # argmax keys (4 slots per request and position) and 4352
    # barrier words (the position barrier's words, then 32 blocks'
    # per-block barriers of 1 KB each),
    # then one (max, sum) pair per chunk, request and position (the fp32
    # path's bound)
    assert ws == 8 * (4 * 128 * 16 + 4352) + 16 * 128 * n_c * 8
    assert B.dspark_workspace_size(B.WS_VERIFY, 128, 16, 129280, 256) >= 4 * 128 * (2 * n_c + 33)
    assert B.dspark_workspace_size(B.WS_SAMPLE, 0, 16, 129280, 256) == 0
    assert B.dspark_workspace_size(B.WS_VERIFY, 4, 0, 1000, 256) == 0
    # the scheduler's ranked slot keys: 8 bytes per slot, rounded up to 256
    assert B.dspark_workspace_size(B.WS_SCHEDULE, 128, 16, 0, 0) == 8 * 128 * 16
    assert B.dspark_workspace_size(B.WS_SCHEDULE, 3, 5, 0, 0) == 256
    assert B.dspark_workspace_size(B.WS_SCHEDULE, 482, 16, 0, 0) == 0   # 482 * 17 > 8191
    # the RNN head adds the hidden-state projection's partials for every
    # (request, position), [splits][R gamma][3r] f32 (bf16 ranks; 4 splits at
    # R gamma = 2048, r = 256: 64 blocks of 256 x 96 fill the compute units
    # four times over), or one position's [R][3r] f32 (fp32 ranks of any size)
    base = B.dspark_workspace_size(B.WS_SAMPLE, 128, 16, 129280, 256)
    base = (base + 255) // 256 * 256
    assert B.dspark_workspace_size(B.WS_RNN_SAMPLE, 128, 16, 129280, 256) == base + 4 * 4 * 2048 * 768
    for r in (1, 20, 33, 1024):
        base = (B.dspark_workspace_size(B.WS_SAMPLE, 9, 7, 333, r) + 255) // 256 * 256
        assert B.dspark_workspace_size(B.WS_RNN_SAMPLE, 9, 7, 333, r) >= base + 4 * 9 * 3 * r


P = ctypes.c_void_p
FAKE = P(0x1000)   # never dereferenced: every call below fails its host checks first


def sample_call(lib, dt=1, R=4, gamma=3, V=1000, r=256, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.dspark_markov_sample(dt, R, gamma, V, r, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                    ws, ws_bytes, None)


def test_sample_rejects_bad_arguments(lib):
    assert sample_call(lib, dt=7) == EDTYPE
    assert sample_call(lib, R=0) == EINVAL
    assert sample_call(lib, gamma=0) == EINVAL
    assert sample_call(lib, gamma=65) == EINVAL
    assert sample_call(lib, V=1) == EINVAL
    assert sample_call(lib, V=1 << 24) == EINVAL
    assert sample_call(lib, r=96) == EDTYPE       # bf16 tile needs 32, 64, 128 or 256
    assert sample_call(lib, r=512) == EDTYPE
    assert sample_call(lib, ptr=None) == EINVAL
    assert sample_call(lib, ws=None) == EWORKSPACE
    assert sample_call(lib, ws_bytes=16) == EWORKSPACE
    assert sample_call(lib, dt=0, r=2000) == EDTYPE


def test_confidence_rejects_bad_arguments(lib):
    def call(dt=1, R=2, gamma=3, d=64, r=32, V=100, ptr=FAKE):
        return lib.dspark_confidence(dt, R, gamma, d, r, V, ptr, ptr, ptr, ptr, ptr, None, ptr, None, None)
    assert call(dt=3) == EDTYPE
    assert call(d=63) == EINVAL
    assert call(r=12) == EINVAL                 # bf16 needs multiples of 8
    assert call(R=0) == EINVAL
    assert call(ptr=None) == EINVAL


def test_schedule_rejects_bad_arguments(lib):
    def call(R=4, gamma=3, n_sps=16, ptr=FAKE):
        return lib.dspark_schedule(R, gamma, ptr, ptr, n_sps, ptr, None, None, None, 0, None)
    assert call(n_sps=15) == EINVAL             # SPS table must reach R * (1 + gamma)
    assert call(R=0) == EINVAL
    assert call(gamma=0) == EINVAL
    assert call(R=482, gamma=16, n_sps=10000) == EINVAL   # 482 * 17 > 8191
    assert call(ptr=None) == EINVAL
    # valid arguments without the workspace (or with too little of it)
    assert call() == EWORKSPACE
    assert lib.dspark_schedule(4, 3, FAKE, FAKE, 16, FAKE, None, None, FAKE, 95, None) == EWORKSPACE


def test_schedule_ex_rejects_bad_arguments(lib):
    def call(R=4, gamma=3, n_sps=16, mode=0, cap=FAKE, ptr=FAKE):
        return lib.dspark_schedule_ex(R, gamma, ptr, ptr, n_sps, mode, cap, ptr, None, None, None, 0, None)
    assert call(mode=3) == EINVAL               # unknown admission rule
    assert call(mode=-1) == EINVAL
    assert call(mode=2, cap=None) == EINVAL     # the capacity rule needs K
    assert call(n_sps=15) == EINVAL
    assert call(R=482, gamma=16, n_sps=10000) == EINVAL
    assert call(ptr=None) == EINVAL
    assert call() == EWORKSPACE


def test_verify_greedy_rejects_bad_arguments(lib):
    def call(dt=1, R=2, gamma=3, V=500, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.dspark_verify_greedy(dt, R, gamma, V, ptr, None, ptr, ptr, ptr, ptr, ws, ws_bytes, None)
    assert call(dt=5) == EDTYPE
    assert call(V=0) == EINVAL
    assert call(gamma=65) == EINVAL
    assert call(ptr=None) == EINVAL
    assert call(ws_bytes=8) == EWORKSPACE


def test_acceptance_rejects_bad_arguments(lib):
    def call(dt=1, R=2, gamma=3, V=500, r=64, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
        a = [ptr] * 8
        return lib.dspark_acceptance(dt, R, gamma, V, r, a[0], None, a[1], a[2], a[3], None, *a[4:], ws, ws_bytes,
                                     None)
    assert call(dt=5) == EDTYPE
    assert call(V=0) == EINVAL
    assert call(r=48) == EDTYPE
    assert call(ptr=None) == EINVAL
    assert call(ws_bytes=8) == EWORKSPACE


def test_rnn_sample_rejects_bad_arguments(lib):
    def call(dt=1, R=2, gamma=3, V=500, r=64, d=32, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
        args = [ptr] * 13
        return lib.dspark_rnn_sample(dt, R, gamma, V, r, d, *args, ws, ws_bytes, None)
    assert call(dt=5) == EDTYPE
    assert call(r=48) == EDTYPE
    assert call(d=24) == EINVAL                 # bf16 hidden size must be a multiple of 16
    assert call(d=0) == EINVAL
    assert call(V=0) == EINVAL
    assert call(ptr=None) == EINVAL
    assert call(ws_bytes=8) == EWORKSPACE


def test_rnn_sample_ex_and_prepare_reject_bad_arguments(lib):
    def call_ex(dt=1, R=2, gamma=3, V=500, r=64, d=32, ptr=FAKE, P=FAKE, ws=FAKE, ws_bytes=1 << 30):
        args = [ptr] * 8 + [P] + [ptr] * 5      # U W1 W2t Wrnn h x0 G g, P, x lse logit s o
        return lib.dspark_rnn_sample_ex(dt, R, gamma, V, r, d, *args, ws, ws_bytes, None)
    assert call_ex(dt=5) == EDTYPE
    assert call_ex(r=48) == EDTYPE
    assert call_ex(d=24) == EINVAL
    assert call_ex(ptr=None) == EINVAL
    assert call_ex(ws_bytes=8) == EWORKSPACE

    def prep(dt=1, V=500, r=64, d=32, W1=FAKE, W=FAKE, P=FAKE):
        return lib.dspark_rnn_prepare(dt, V, r, d, W1, W, P, None)
    assert prep(dt=0) == EDTYPE                 # the table is made for bf16 weights only
    assert prep(dt=5) == EDTYPE
    assert prep(r=48) == EDTYPE
    assert prep(V=1) == EINVAL
    assert prep(V=1 << 24) == EINVAL
    assert prep(d=24) == EINVAL
    assert prep(W1=None) == EINVAL
    assert prep(P=None) == EINVAL


def test_sts_fit_rejects_bad_arguments(lib):
    def call(N=100, gamma=4, G=16, M=15, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return lib.dspark_sts_fit(N, gamma, ptr, ptr, ptr, G, M, ptr, ptr, ptr, ptr, ws, ws_bytes, None)
    assert call(N=0) == EINVAL
    assert call(N=(1 << 20) + 1) == EINVAL
    assert call(G=257) == EINVAL
    assert call(M=33) == EINVAL
    assert call(gamma=65) == EINVAL
    assert call(ptr=None) == EINVAL
    assert call(ws_bytes=8) == EWORKSPACE


def test_verify_ex_rejects_bad_arguments(lib):
    def call(dt=1, R=2, gamma=3, V=500, r=64, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
        a = [ptr] * 13
        return lib.dspark_verify_ex(dt, R, gamma, V, r, a[0], None, a[1], a[2], a[3], ptr, *a[4:], ws, ws_bytes,
                                    None)
    assert call(dt=5) == EDTYPE
    assert call(V=0) == EINVAL
    assert call(r=48) == EDTYPE
    assert call(ptr=None) == EINVAL
    assert call(ws_bytes=8) == EWORKSPACE


def test_verify_rejects_bad_arguments(lib):
    def call(dt=1, R=2, gamma=3, V=500, r=64, ptr=FAKE, ws=FAKE, ws_bytes=1 << 30):
        args = [ptr] * 13
        return lib.dspark_verify(dt, R, gamma, V, r, args[0], None, *args[1:], ws, ws_bytes, None)
    assert call(dt=5) == EDTYPE
    assert call(V=0) == EINVAL
    assert call(r=48) == EDTYPE
    assert call(ptr=None) == EINVAL
    assert call(ws_bytes=8) == EWORKSPACE


def test_sample_ex_rejects_bad_arguments(lib):
    def call(dt=1, R=4, gamma=3, V=1000, r=256, d=64, ptr=FAKE, h=FAKE, w=FAKE, c=FAKE, ws=FAKE,
             ws_bytes=1 << 30, events=None):
        a = [ptr] * 6
        return lib.dspark_markov_sample_ex(dt, R, gamma, V, r, d, *a, h, w, None, ptr, ptr, ptr, c, None,
                                           None, None, events, ws, ws_bytes, None)
    assert call(dt=7) == EDTYPE
    assert call(R=0) == EINVAL
    assert call(r=96) == EDTYPE
    assert call(ptr=None) == EINVAL
    assert call(w=None) == EINVAL               # the confidence head needs its weights
    assert call(c=None) == EINVAL               # ... and somewhere to put c
    assert call(d=60) == EINVAL                 # bf16 hidden size: a multiple of 8
    assert call(events=(ctypes.c_void_p * 2)(FAKE, None)) == EINVAL   # both events or none
    assert call(ws=None) == EWORKSPACE
    # without the confidence head its arguments are ignored
    assert call(h=None, w=None, c=None, d=0, ws=None) == EWORKSPACE


def test_schedule_noalloc_rejects_bad_arguments(lib):
    def call(R=4, gamma=3, n_sps=16, mode=0, cap=FAKE, ptr=FAKE):
        return lib.dspark_schedule_noalloc(R, gamma, ptr, ptr, n_sps, mode, cap, ptr, None, None, None)
    assert call(mode=3) == EINVAL
    assert call(mode=2, cap=None) == EINVAL
    assert call(n_sps=15) == EINVAL
    assert call(R=482, gamma=16, n_sps=10000) == EINVAL   # beyond the static scratch
    assert call(R=0) == EINVAL
    assert call(ptr=None) == EINVAL


def test_sample_kernel_query_rejects_what_the_call_rejects(lib):
    # the same host checks as the sampling call: NULL for a bad type, shape
    # or rank, and (on a machine without a gfx950 device) for valid ones too
    assert lib.dspark_markov_sample_kernel(7, 128, 16, 129280, 256) is None
    assert lib.dspark_markov_sample_kernel(1, 0, 16, 129280, 256) is None
    assert lib.dspark_markov_sample_kernel(1, 128, 16, 129280, 96) is None
    assert lib.dspark_rnn_sample_kernel(7, 128, 16, 129280, 256) is None
    assert lib.dspark_rnn_sample_kernel(1, 0, 16, 129280, 256) is None
    assert lib.dspark_rnn_sample_kernel(1, 128, 16, 129280, 96) is None
