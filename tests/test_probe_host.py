"""The benchmark's HBM stream probe on the host: libkvsel_probe.so loads,
exports its one entry point (and libkvsel.so does not), and it rejects bad
arguments before enqueuing anything."""
import sparse_decode_attention_window_amd as kvsel
from sparse_decode_attention_window_amd import _probe as probe

FAKE = 0x1000   # never dereferenced: every call below fails its host checks first


def test_probe_is_outside_the_method_library():
    assert hasattr(probe.lib(), "kvsel_probe_stream")
    assert not hasattr(kvsel.lib(), "kvsel_hbm_probe")
    assert not hasattr(kvsel.lib(), "kvsel_probe_stream")


def test_hbm_probe_rejects_bad_arguments():
    """Mode, pointers, alignment and size are checked on the host; nothing is
    enqueued when a check fails (status 1)."""
    fn = probe.lib().kvsel_probe_stream
    ok_src, ok_dst = FAKE, FAKE + 0x100000
    cases = [
        (2, ok_src, ok_dst, 1024),          # unknown mode
        (-1, ok_src, ok_dst, 1024),
        (0, None, ok_dst, 1024),            # NULL source
        (1, ok_src, None, 1024),            # NULL destination
        (1, ok_src + 8, ok_dst, 1024),      # misaligned source
        (0, ok_src, ok_dst + 4, 1024),      # misaligned destination
        (1, ok_src, ok_dst, 0),             # empty
        (1, ok_src, ok_dst, -16),
        (0, ok_src, ok_dst, 1000),          # not a multiple of 16
    ]
    for mode, src, dst, nbytes in cases:
        assert fn(mode, src, dst, nbytes, None) == 1, (mode, src, dst, nbytes)
    assert probe.PROBE_BLOCKS == 2048
