"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device (CPU only)."""
import ctypes
import os
import re
import subprocess

import pytest

import distance_geometry_bound_amd as dgb
from distance_geometry_bound_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dbs.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dbs_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = dgb.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (DBS_[A-Z_]+) \(?(-?\d+)u?\)?", text))
    assert int(consts["DBS_OK"]) == _lib.DBS_OK
    assert int(consts["DBS_EINVAL"]) == _lib.DBS_EINVAL
    assert int(consts["DBS_EDEVICE"]) == _lib.DBS_EDEVICE
    assert int(consts["DBS_ELAUNCH"]) == _lib.DBS_ELAUNCH
    assert int(consts["DBS_EUNSUPPORTED"]) == _lib.DBS_EUNSUPPORTED
    assert int(consts["DBS_ALGO_PERK"]) == _lib.ALGO_PERK
    assert int(consts["DBS_ALGO_LDS"]) == _lib.ALGO_LDS
    assert int(consts["DBS_ALGO_BLOCKED"]) == _lib.ALGO_BLOCKED
    for k, v in _lib.CHECK_FLAGS.items():
        assert int(consts["DBS_CHECK_" + k.upper().replace("NONFINITE", "NONFINITE")]) == v


def test_static_queries():
    L = dgb.lib()
    assert L.dbs_version() == 0x000100
    assert L.dbs_lds_max_n() >= 128
    assert L.dbs_auto_algo(127, 1) == _lib.ALGO_LDS
    assert L.dbs_auto_algo(128, 1) == _lib.ALGO_BLOCKED
    assert L.dbs_auto_algo(176, 16) == _lib.ALGO_BLOCKED
    assert L.dbs_auto_algo(128, 17) == _lib.ALGO_LDS
    assert L.dbs_auto_algo(176, 64) == _lib.ALGO_LDS
    assert L.dbs_auto_algo(177, 64) == _lib.ALGO_BLOCKED
    assert L.dbs_auto_algo(12288, 1) == _lib.ALGO_BLOCKED
    assert L.dbs_strerror(-1) == b"invalid argument"
    assert L.dbs_strerror(12345) == b"unknown status"


# host-side argument validation: fake, never dereferenced addresses.  These
# cases run only where no GPU is visible: with a GPU, a regression in the
# order of the checks could launch a kernel on them.
A, B = 0x10000000, 0x20000000


@pytest.fixture
def no_gpu():
    import torch

    if torch.cuda.is_available():
        pytest.skip("fake device addresses are only passed where no GPU is visible")


@pytest.mark.parametrize("args", [
    (0, B, 4, 1), (A, 0, 4, 1), (A, B, 0, 1), (A, B, -3, 1), (A, B, 4, 0),
    (A, B, 1 << 31, 1), (A, A + (1 << 55), 1 << 26, 1),  # 2^26: the size limit alone
    (A, B, 1 << 20, 1 << 40), (A, A + 32, 4, 1), (A + 2, B, 4, 1),
])
def test_smooth_rejects_bad_arguments(args, no_gpu):
    L = dgb.lib()
    assert L.dbs_smooth(*args, None) == _lib.DBS_EINVAL
    assert L.dbs_smooth_algo(*args, None, 0) == _lib.DBS_EINVAL


def test_rounds_and_algo_range_checks(no_gpu):
    L = dgb.lib()
    assert L.dbs_rounds(A, B, 8, 1, 5, 4, None) == _lib.DBS_EINVAL
    assert L.dbs_rounds(A, B, 8, 1, -1, 4, None) == _lib.DBS_EINVAL
    assert L.dbs_rounds(A, B, 8, 1, 0, 9, None) == _lib.DBS_EINVAL
    assert L.dbs_smooth_algo(A, B, 8, 1, None, 7) == _lib.DBS_EINVAL
    assert L.dbs_smooth_algo(A, B, 1000, 1, None, _lib.ALGO_LDS) == _lib.DBS_EUNSUPPORTED
    assert L.dbs_check(A, B, 8, 1, None, None) == _lib.DBS_EINVAL     # null d_flags
    assert L.dbs_check(A, B, 0, 1, None, A + 64) == _lib.DBS_EINVAL
    assert L.dbs_check_packed(A, 8, 1, None, None) == _lib.DBS_EINVAL


def test_options_are_validated_on_the_host(no_gpu):
    L = dgb.lib()
    byref = ctypes.byref
    good = _lib.Options(0, 0, -1, -1, -1)
    d = _lib.Options(9, 9, 9, 9, 9, A)
    L.dbs_options_init(byref(d))
    assert (d.algo, d.directed, d.lookahead, d.step_blocks, d.lead) == (0, 0, -1, -1, -1)
    assert d.infeasible is None
    for bad in (_lib.Options(4, 0, -1, -1, -1), _lib.Options(-1, 0, -1, -1, -1),
                _lib.Options(0, 2, -1, -1, -1), _lib.Options(0, 0, 3, -1, -1),
                _lib.Options(0, 0, -2, -1, -1), _lib.Options(0, 0, -1, 0, -1),
                _lib.Options(0, 0, -1, 5, -1), _lib.Options(0, 0, -1, -1, 2),
                _lib.Options(0, 0, -1, -1, -2), _lib.Options(0, 0, -1, -1, -1, A + 2)):
        assert L.dbs_smooth_opts(A, B, 8, 1, 0, 8, None, byref(bad)) == _lib.DBS_EINVAL
        assert L.dbs_smooth_packed_opts(A, 8, 1, 0, 8, None, byref(bad)) == _lib.DBS_EINVAL
        assert L.dbs_schedule(8, 1, byref(bad), None, None, None) == _lib.DBS_EINVAL
    # blocked ranges must start and end on k-block boundaries
    blk = _lib.Options(_lib.ALGO_BLOCKED, 0, -1, -1, -1)
    assert L.dbs_smooth_opts(A, B, 300, 1, 0, 100, None, byref(blk)) == _lib.DBS_EUNSUPPORTED
    assert L.dbs_smooth_packed_opts(A, 300, 1, 64, 100, None, byref(blk)) == \
        _lib.DBS_EUNSUPPORTED
    lds = _lib.Options(_lib.ALGO_LDS, 0, -1, -1, -1)
    assert L.dbs_smooth_packed_opts(A, 300, 1, 0, 300, None, byref(lds)) == \
        _lib.DBS_EUNSUPPORTED
    assert L.dbs_smooth_opts(A, B, 8, 1, 5, 4, None, byref(good)) == _lib.DBS_EINVAL
    assert L.dbs_smooth_opts(A, A + 16, 8, 1, 0, 8, None, byref(good)) == _lib.DBS_EINVAL
    counts = (ctypes.c_int64 * len(_lib.PROF_KINDS))()
    ms = (ctypes.c_double * len(_lib.PROF_KINDS))()
    assert L.dbs_smooth_profiled(A, B, 8, 1, None, byref(good), None, ms) == _lib.DBS_EINVAL
    assert L.dbs_smooth_profiled(A, B, 8, 1, None, byref(d), counts, None) == _lib.DBS_EINVAL


def test_options_layout_matches_the_header(tmp_path):
    # the binding's struct dbs_options against the C compiler's
    src = tmp_path / "layout.c"
    src.write_text('#include "dbs.h"\n#include <stddef.h>\n#include <stdio.h>\n'
                   'int main(void) { printf("%zu %zu %zu\\n", sizeof(dbs_options), '
                   'offsetof(dbs_options, lead), offsetof(dbs_options, infeasible)); '
                   'return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe)], check=True)
    got = tuple(int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                               text=True).stdout.split())
    assert got == (ctypes.sizeof(_lib.Options), _lib.Options.lead.offset,
                   _lib.Options.infeasible.offset)


def test_no_device_is_reported(no_gpu):
    L = dgb.lib()
    assert L.dbs_smooth(A, B, 8, 1, None) == _lib.DBS_EDEVICE
    assert L.dbs_rounds(A, B, 8, 1, 0, 1, None) == _lib.DBS_EDEVICE
    assert L.dbs_smooth_opts(A, B, 8, 1, 0, 8, None, None) == _lib.DBS_EDEVICE


def test_python_wrapper_rejects_cpu_tensors():
    import torch

    U = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        dgb.smooth(U, U.clone())
    with pytest.raises(TypeError):
        dgb.smooth(U.double(), U.double())


def test_round_rejects_k_out_of_range_on_the_host():
    # argument errors are found before anything is enqueued (no device needed)
    import ctypes
    lib = dgb.lib()
    buf = (ctypes.c_float * 16)()
    p = ctypes.cast(buf, ctypes.c_void_p).value
    assert lib.dbs_round(p, p, 4, 1, -1, None) == -1
    assert lib.dbs_round(p, p, 4, 1, 4, None) == -1


def test_lookahead_bands_query():
    # host-side shape logic only (no device call)
    lib = dgb.lib()
    assert lib.dbs_lookahead_bands(1, 1) == 0        # nothing to run ahead
    assert lib.dbs_lookahead_bands(64, 1) == 0       # one k-block
    assert lib.dbs_lookahead_bands(128, 3) == 0      # one phase-3 tile
    assert lib.dbs_lookahead_bands(200, 1) == 0       # 3 tiles: bulk shorter than a strip
    assert lib.dbs_lookahead_bands(1024, 1) == 0      # 36 tiles
    assert lib.dbs_lookahead_bands(500, 64) == 0      # 448 panel workgroups fill the chip
    assert lib.dbs_lookahead_bands(130, 129) == 0     # 387 tiles, a batch: the lead schedule
    assert lib.dbs_lookahead_bands(130, 128) == 0     # 384 tiles: the lead schedule
    assert lib.dbs_lookahead_bands(2944, 1) == 0      # 276 tiles: the lead schedule
    assert lib.dbs_lookahead_bands(4096, 1) == 1
    assert lib.dbs_lookahead_bands(4864, 1) == 1      # 741 tiles
    assert lib.dbs_lookahead_bands(5120, 1) == 2      # 820 tiles, one molecule
    assert lib.dbs_lookahead_bands(5632, 1) == 2      # 990 tiles
    assert lib.dbs_lookahead_bands(2048, 4) == 0      # 544 tiles, a batch: the lead schedule
    assert lib.dbs_lookahead_bands(1024, 28) == 0     # 1008 tiles, a batch
    assert lib.dbs_lookahead_bands(6144, 1) == 2      # 1176 tiles
    assert lib.dbs_lookahead_bands(4096, 2) == 2      # 1056 tiles x molecules
    assert lib.dbs_lookahead_bands(12288, 1) == 2
    assert lib.dbs_lookahead_bands(0, 1) == -1 and lib.dbs_lookahead_bands(5, 0) == -1
    assert dgb.lookahead_bands(12288) == 2


def test_schedule_query_with_forced_values():
    # a forced depth or width applies to that call's options only; the
    # library keeps no setting between calls
    assert dgb.schedule(200, lookahead=2) == (2, 2, 0)
    assert dgb.schedule(4096, lookahead=2)[0] == 2
    assert dgb.schedule(64, lookahead=2)[0] == 0 and dgb.schedule(128, 3, lookahead=2)[0] == 0
    assert dgb.schedule(12288, lookahead=0) == (0, 1, 0)
    assert dgb.schedule(12288) == (2, 4, 0) and dgb.schedule(200) == (0, 1, 0)
    assert dgb.schedule(200, step_blocks=4) == (0, 4, 0)
    assert dgb.schedule(12288, lookahead=1, step_blocks=3) == (1, 3, 0)
    # the lead schedule: automatic for a batch from 64 to 1023 phase-3 tiles
    # (128-atom tiles I <= J, times molecules), for one molecule from 64 to
    # 511; forced on any one-stream pass with one-block steps
    assert dgb.schedule(500, 64) == (0, 1, 1) and dgb.schedule(130, 129) == (0, 1, 1)
    assert dgb.schedule(300, 100) == (0, 1, 1)               # 600 tiles, 400 panel tiles
    assert dgb.schedule(300, 100, lead=False) == (0, 1, 0)   # the split batch instead
    assert dgb.schedule(1024)[2] == 0 and dgb.schedule(1280) == (0, 1, 0)   # 36, 55 tiles
    assert dgb.schedule(500, 4) == (0, 1, 0)                 # 40 tiles
    assert dgb.schedule(500, 8) == (0, 1, 1) and dgb.schedule(1792) == (0, 1, 1)  # 80, 105
    assert dgb.schedule(2048) == (0, 1, 1) and dgb.schedule(3072) == (0, 1, 1)  # 136, 300
    assert dgb.schedule(500, 16) == (0, 1, 1) and dgb.schedule(130, 128) == (0, 1, 1)
    assert dgb.schedule(4096) == (1, 1, 0)                   # 528 tiles: one step ahead
    assert dgb.schedule(4864) == (1, 1, 0)                   # 741 tiles
    assert dgb.schedule(5120) == (2, 1, 0)                   # 820: two ahead, one-block steps
    assert dgb.schedule(6144) == (2, 2, 0)                   # 1176 tiles
    assert dgb.schedule(1024, 16) == (0, 1, 1) and dgb.schedule(2048, 4) == (0, 1, 1)
    assert dgb.schedule(3072, 2) == (0, 1, 1) and dgb.schedule(2048, 6) == (0, 1, 1)
    assert dgb.schedule(500, 128) == (2, 1, 0)               # a batch, 1280 tiles
    assert dgb.schedule(1024, 64) == (2, 2, 0)               # 2304 tiles
    assert dgb.schedule(500, 512) == (2, 4, 0)               # 5120 tiles
    assert dgb.schedule(128, 1200) == (0, 1, 1)              # one tile each: never ahead
    assert dgb.schedule(3072, lead=False) == (1, 1, 0)
    # the packed layout takes the lead window from 256 tiles
    assert dgb.schedule(1536, packed=True) == (0, 1, 0)      # 78 tiles
    assert dgb.schedule(2048, packed=True) == (0, 1, 0)      # 136 tiles
    assert dgb.schedule(2560, packed=True) == (0, 1, 0)      # 210 tiles
    assert dgb.schedule(3072, packed=True) == (0, 1, 1)      # 300 tiles
    assert dgb.schedule(500, 64, packed=True) == (0, 1, 1)   # the panel launch fills the chip
    assert dgb.schedule(4096, packed=True) == (1, 1, 0)
    assert dgb.schedule(5120, packed=True) == (1, 1, 0)      # the dense rules above only
    assert dgb.schedule(2048, 4, packed=True) == (1, 1, 0)
    assert dgb.schedule(500, 128, packed=True) == (2, 2, 0)
    assert dgb.schedule(12288, packed=True) == (2, 4, 0)
    assert dgb.schedule(1536, packed=True, lead=True) == (0, 1, 1)
    assert dgb.schedule(500, 64, lead=False) == (0, 1, 0)
    assert dgb.schedule(1024, lead=True) == (0, 1, 1)
    assert dgb.schedule(12288, lead=True) == (2, 4, 0)        # runs ahead: no lead
    assert dgb.schedule(1024, lead=True, step_blocks=2) == (0, 2, 0)
    assert dgb.schedule(64, lead=True)[2] == 0                 # one k-block
    for la, sb, ld in ((3, None, None), (-2, None, None), (None, 0, None), (None, 5, None),
                       (None, None, 2)):
        with pytest.raises(ValueError):
            dgb.schedule(12288, lookahead=la, step_blocks=sb, lead=ld)
    lib = dgb.lib()
    la, sb, ld = ctypes.c_int32(7), ctypes.c_int32(7), ctypes.c_int32(7)
    assert lib.dbs_schedule(12288, 1, None, ctypes.byref(la), ctypes.byref(sb),
                            ctypes.byref(ld)) == 0
    assert (la.value, sb.value, ld.value) == (2, 4, 0)
    assert lib.dbs_schedule(0, 1, None, None, None, None) == -1
    assert lib.dbs_schedule(5, 0, None, None, None, None) == -1
    assert lib.dbs_schedule(5, 1, None, None, None, None) == 0


def test_step_blocks_query():
    # steps of several k-blocks where the pass runs two steps ahead, else one
    lib = dgb.lib()
    assert dgb.step_blocks(12288) == 4 and dgb.step_blocks(10240) == 4   # 4656, 3240 tiles
    assert dgb.step_blocks(8192) == 3 and dgb.step_blocks(6144, 2) == 2  # 2080, 2352
    assert dgb.step_blocks(500, 128) == 1 and dgb.step_blocks(1024, 64) == 2  # 1280, 2304
    assert dgb.step_blocks(5632) == 1 and dgb.step_blocks(6144) == 2     # 990, 1176
    assert dgb.step_blocks(4096) == 1 and dgb.step_blocks(200) == 1
    assert lib.dbs_step_blocks(0, 1) == -1 and lib.dbs_step_blocks(5, 0) == -1
