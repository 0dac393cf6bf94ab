"""Host-side choices of the layer schedules (no GPU)."""
import pytest

from decode_focal_layer_amd.decode import shared_parts


@pytest.mark.parametrize("query_rows,hkv,rows,per_cu,want", [
    (512 * 8 * 2, 8, 1024, 1, 1),      # draft verification: 8192 query rows per kv head already fill the chip
    (512 * 2, 8, 1024, 1, 4),          # branched decode, sparse layers: 64 work-groups -> 4 parts
    (512 * 2, 8, 4096, 2, 8),          # focal layers (logits pass): two work-groups per CU
    (10, 2, 100, 1, 1),                # a range shorter than two tiles stays whole
    (2, 1, 1 << 20, 1, 64),            # never more than 64 parts
    (2, 1, 300, 1, 2),                 # at least two 64-row tiles per part
])
def test_shared_parts(query_rows, hkv, rows, per_cu, want):
    assert shared_parts(query_rows, hkv, rows, per_cu) == want
