"""Host-side argument checks of the torch API (no GPU and no library call needed)."""
import pytest
import torch

from kl_knowledge_distillation_amd import api


def _cpu_problem():
    h = torch.zeros(4, 8)
    w = torch.zeros(16, 8)
    return h, w, torch.zeros(4, dtype=torch.int64)


def test_unknown_kl_divergence_is_rejected():
    h, w, y = _cpu_problem()
    with pytest.raises(ValueError, match="kl_divergence"):
        api.distillation_loss(h, w, y, api.TiedTeacher(h), kl_divergence="js")


@pytest.mark.parametrize("kl", ["reverse", "jeffreys"])
def test_topk_teacher_allows_forward_kl_only(kl):
    h, w, _ = _cpu_problem()
    t = api.TopKTeacher(torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2))
    with pytest.raises(NotImplementedError, match="top-K"):
        api.distillation_loss(h, w, None, t, kl_weight=1.0, kl_divergence=kl)


def test_kl_divergence_table_matches_the_header():
    from kl_knowledge_distillation_amd import _lib as L
    assert api._KL_DIVERGENCES == {"forward": L.KD_KL_FORWARD, "reverse": L.KD_KL_REVERSE,
                                   "jeffreys": L.KD_KL_JEFFREYS}
    assert (L.KD_KL_FORWARD, L.KD_KL_REVERSE, L.KD_KL_JEFFREYS) == (0, 1, 2)


def test_precomputed_teacher_takes_one_form():
    x = torch.zeros(4, 16)
    h, w = torch.zeros(4, 8), torch.zeros(16, 8)
    api.PrecomputedTeacher(logits=x)
    api.PrecomputedTeacher(teacher_hidden=h, teacher_weight=w)
    for bad in (dict(), dict(logits=x, teacher_hidden=h, teacher_weight=w), dict(teacher_hidden=h)):
        with pytest.raises(ValueError):
            api.PrecomputedTeacher(**bad)


def test_teacher_temperature_must_be_positive():
    h, w, y = _cpu_problem()
    with pytest.raises(ValueError, match="kl_teacher_temperature"):
        api.distillation_loss(h, w, y, api.TiedTeacher(h), kl_teacher_temperature=0.0)


def test_compact_valid_needs_labels_and_a_projected_teacher():
    h, w, y = _cpu_problem()
    t = api.TopKTeacher(torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2))
    with pytest.raises(NotImplementedError, match="compact_valid"):
        api.distillation_loss(h, w, None, t, kl_weight=1.0, student_ce_weight=0.0, compact_valid=True)
    with pytest.raises(NotImplementedError, match="compact_valid"):
        api.distillation_loss(h, w, y, api.PrecomputedTeacher(logits=torch.zeros(4, 16)),
                              compact_valid=True)


def test_tied_teacher_mode_asserts_the_role():
    h, w, y = _cpu_problem()
    with pytest.raises(ValueError, match="frozen"):
        api.distillation_loss(h, w, y, api.TiedTeacher(h, mode="trained"), teacher_ce_weight=0.0)
    with pytest.raises(ValueError, match="trained"):
        api.distillation_loss(h, w, y, api.TiedTeacher(h, mode="frozen"), teacher_ce_weight=1.0)
    with pytest.raises(NotImplementedError):
        api.distillation_loss(h, w, y, api.TiedTeacher(h, mode="cotrained"))


def test_precomputed_teacher_must_not_require_grad():
    h, w, y = _cpu_problem()
    t = api.PrecomputedTeacher(logits=torch.zeros(4, 16, requires_grad=True))
    with pytest.raises(ValueError, match="require grad"):
        api.distillation_loss(h, w, y, t)


def test_kdloss_rejects_mixed_dtypes_instead_of_casting():
    """An fp32 teacher with a bf16 student is an error, not a silent rounding."""
    z = torch.zeros(4, 16, dtype=torch.bfloat16)
    t = torch.zeros(4, 16, dtype=torch.float32)
    with pytest.raises(TypeError, match="dtype"):
        api.KDLoss()(z, t, torch.zeros(4, dtype=torch.int64))
