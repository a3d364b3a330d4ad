"""Host-side checks of the layer-stream driver: shapes are validated before any
library call, and the reused storage has the sizes of the storage format."""
import pytest

import oracle
from qlora_linear_layers_amd.stream import LayerStream


def test_storage_sizes_match_the_format():
    st = LayerStream([(1024, 8192), (8192, 28672)], device="cpu")
    for (N, K), qw, wd in zip(st.shapes, st.qws, st.wds):
        assert qw.nbytes() == oracle.storage_bytes(N * K)
        assert tuple(wd.shape) == (N, K)


def test_rejects_bad_shapes_before_any_call():
    import torch
    st = LayerStream([(64, 128)], device="cpu")
    with pytest.raises(ValueError):
        st.run(lambda l: [torch.zeros((128, 64), dtype=torch.bfloat16)], 1, timed=False)
    with pytest.raises(ValueError):
        st.run(lambda l: [], 1, timed=False)
    with pytest.raises(ValueError):
        LayerStream([(3, 7)], device="cpu")
