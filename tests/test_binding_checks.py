"""The binding refuses, before any pointer reaches the library, tensors the C
ABI would misread (the library sees raw pointers and cannot check sizes,
dtypes or devices), and checks a host copy of a slot table on request. CPU
only: no call here reaches the library."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from linear_attention_verify_amd import binding as bd  # noqa: E402
from linear_attention_verify_amd import workloads as wl  # noqa: E402


@pytest.fixture
def no_library(monkeypatch):
    """Any call that gets as far as the library fails the test."""
    def refuse(*a, **k):
        raise AssertionError("the library was reached")
    monkeypatch.setattr(bd, "load_library", refuse)


def test_check_refuses_wrong_dtype():
    with pytest.raises(ValueError, match="int32"):
        bd._check(torch.zeros(4, dtype=torch.int64), "slot_ids", torch.int32, (4,))


def test_check_refuses_wrong_shape_and_size():
    with pytest.raises(ValueError, match="shape"):
        bd._check(torch.zeros(2, 3, 5), "x", torch.float32, (2, 3, 4))
    with pytest.raises(ValueError, match="shape"):
        bd._check(torch.zeros(2, 3), "x", torch.float32, (2, 3, 1))
    with pytest.raises(ValueError, match="at least"):
        bd._check(torch.zeros(0, dtype=torch.int32), "err_flag", torch.int32, min_numel=1)


def test_check_refuses_non_contiguous():
    t = torch.zeros(4, 6)[:, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        bd._check(t, "x", torch.float32)


def test_check_refuses_host_memory_and_non_tensors():
    with pytest.raises(ValueError, match="GPU memory"):
        bd._check(torch.zeros(4, dtype=torch.int32), "slot_ids", torch.int32, (4,))
    with pytest.raises(TypeError):
        bd._check(np.zeros(4, np.int32), "slot_ids", torch.int32, (4,))
    with pytest.raises(ValueError, match="required"):
        bd._check(None, "x", torch.float32)
    bd._check(None, "err_flag", torch.int32, optional=True)


def _host_case(dtype="bf16"):
    s = wl.LayerShape(num_k_heads=2, num_v_heads=4, d_k=32, d_v=32, dtype=dtype)
    st = torch.float32 if dtype == "f32" else torch.bfloat16
    B, R, P, C = 3, 4, 5, s.conv_channels
    t = dict(ssm=torch.zeros(P, 4, 32, 32), conv=torch.zeros(P, 3, C, dtype=st),
             conv_w=torch.zeros(C, 4, dtype=st), x=torch.zeros(B, R, C, dtype=st),
             alpha=torch.zeros(B, R, 4, dtype=st), beta=torch.zeros(B, R, 4, dtype=st),
             slot_ids=torch.zeros(B, dtype=torch.int32), accept=torch.zeros(B, dtype=torch.int32),
             scratch=torch.zeros(64, dtype=torch.uint8), out=torch.zeros(B, R, 4, 32, dtype=st),
             err=torch.zeros(1, dtype=torch.int32))
    return bd.layer_desc(s), R, t


def test_verify_and_commit_refuse_host_tensors(no_library):
    desc, R, t = _host_case()
    with pytest.raises(ValueError, match="GPU memory"):
        bd.gdn_spec_verify(desc, t["ssm"], t["conv"], t["conv_w"], t["x"], t["alpha"], t["beta"], t["slot_ids"],
                           R, "replay", t["scratch"], t["out"], t["err"])
    with pytest.raises(ValueError, match="GPU memory"):
        bd.gdn_spec_commit(desc, t["ssm"], t["conv"], t["slot_ids"], t["accept"], R, "replay", t["scratch"],
                           t["err"])
    with pytest.raises(ValueError, match="GPU memory"):
        bd.Prepared(desc, t["ssm"], t["conv"], t["conv_w"], t["x"], t["alpha"], t["beta"], t["slot_ids"],
                    t["accept"], R, "replay", t["scratch"], t["out"], t["err"])


def test_pool_of_the_wrong_layout_is_refused(no_library):
    desc, R, t = _host_case()
    with pytest.raises(ValueError, match="ssm"):          # d_k and d_v swapped for a 64-wide head
        bd.gdn_spec_commit(desc, torch.zeros(5, 4, 32, 64), t["conv"], t["slot_ids"], t["accept"], R,
                           "replay", t["scratch"])
    with pytest.raises(ValueError, match="ssm must be torch.float32"):
        bd.gdn_spec_commit(desc, t["ssm"].double(), t["conv"], t["slot_ids"], t["accept"], R, "replay",
                           t["scratch"])


def test_accept_and_attention_refuse_host_tensors(no_library):
    B, R = 3, 4
    i32 = dict(dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU memory"):
        bd.gdn_spec_accept_greedy(torch.zeros(B, R - 1, **i32), torch.zeros(B, R, **i32), None, R,
                                  torch.zeros(B, **i32))
    with pytest.raises(ValueError, match="int32"):
        bd.gdn_spec_accept_greedy(torch.zeros(B, R - 1, **i32), torch.zeros(B, R, dtype=torch.int64), None, R,
                                  torch.zeros(B, **i32))
    desc = bd.GdnAttnDesc(8, 2, 128, 32, 0.088)
    bf = dict(dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        bd.gdn_spec_attn_verify(desc, torch.zeros(B, R, 8, 128, **bf), torch.zeros(6, 32, 2, 128, **bf),
                                torch.zeros(6, 32, 2, 128, **bf), torch.zeros(B, 2, **i32), torch.zeros(B, **i32),
                                torch.zeros(64, dtype=torch.uint8), torch.zeros(B, R, 8, 128, **bf))


def test_host_slot_table_check():
    bd.check_slot_ids_host([3, -1, 0, 7], 8)
    bd.check_slot_ids_host(np.array([], np.int32), 8)
    bd.check_slot_ids_host(torch.tensor([1, 2, -1, -1], dtype=torch.int32), 3)   # padding may repeat
    with pytest.raises(ValueError, match="shared by requests \\[0, 2\\]"):
        bd.check_slot_ids_host([4, 1, 4], 8)
    with pytest.raises(ValueError, match="outside"):
        bd.check_slot_ids_host([0, 8], 8)
    with pytest.raises(ValueError, match="outside"):
        bd.check_slot_ids_host([0, -2], 8)
    with pytest.raises(ValueError):
        bd.check_slot_ids_host([[0, 1]], 8)


def test_duplicate_slots_stop_the_call_before_the_library(no_library, monkeypatch):
    """With host_slot_ids given, the binding checks it after the tensors; the
    tensor checks are skipped here so that the slot check is what refuses."""
    desc, R, t = _host_case()
    monkeypatch.setattr(bd, "_check_commit_args", lambda *a, **k: 3)
    with pytest.raises(ValueError, match="shared"):
        bd.gdn_spec_commit(desc, t["ssm"], t["conv"], t["slot_ids"], t["accept"], R, "replay", t["scratch"],
                           host_slot_ids=[2, 0, 2])


def test_commit_verify_refuses_host_tensors_and_bad_tables(no_library):
    """The commit-verify's extra tables (source rows, the previous slot table
    and accept lengths) are checked like the others; a host copy of the
    source-row table is checked for range and for a previous row named twice."""
    desc, R, t = _host_case()
    i32 = dict(dtype=torch.int32)
    args = (desc, t["ssm"], t["conv"], t["conv_w"], t["x"], t["alpha"], t["beta"], t["slot_ids"], R, t["scratch"])
    with pytest.raises(ValueError, match="GPU memory"):
        bd.gdn_spec_commit_verify(*args, torch.zeros(3, **i32), t["scratch"], torch.zeros(2, **i32),
                                  torch.zeros(2, **i32), t["out"], t["err"])
    bd.check_src_rows_host([1, -1, 0], 2)
    bd.check_src_rows_host(np.array([], np.int64), 0)
    with pytest.raises(ValueError, match="named by requests \\[0, 2\\]"):
        bd.check_src_rows_host([1, -1, 1], 2)
    with pytest.raises(ValueError, match="outside"):
        bd.check_src_rows_host([2], 2)
    with pytest.raises(ValueError, match="outside"):
        bd.check_src_rows_host([-3], 2)
    with pytest.raises(ValueError):
        bd.check_src_rows_host(torch.zeros(2, dtype=torch.float32), 2)
    bd.check_src_rows_host([1, 1, 0], 2, slot_ids=[4, -1, 5])        # a padding request's source is ignored
    with pytest.raises(ValueError, match="differ in length"):
        bd.check_src_rows_host([1, 0], 2, slot_ids=[4])
