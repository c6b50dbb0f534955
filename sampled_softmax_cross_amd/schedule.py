"""Host-side schedule of the sampled-softmax training loss, for a training loop that
calls the step ("sampled_softmax.py": module docstring on the schedule, the
per-stage candidate counts, `candidate_count_at`, `CandidateBuilder.reset`).

* Which P a step uses: stages 0 and 1 run P = 10240; stage 2 runs 14336, 14336 and
  24576 over equal thirds of its steps; every later stage runs the full softmax
  (P = 0).
* Where a data-parallel rank starts its sweep of k * stride mod V: rank r of `world`
  starts at V * r // world, so the ranks draw different negatives. Later offsets come
  from the step itself (`aux_out[2]`, the offset after the call's window).
"""

# Candidate counts by stage index; a stage with n counts splits its steps into n
# equal parts, one count each. A stage not listed runs the full softmax.
P_BY_STAGE = {0: (10240,), 1: (10240,), 2: (14336, 14336, 24576)}

# The sweep stride (coprime with the 50304-class vocabulary).
SWEEP_STRIDE = 20011


def stage_of(boundaries, step):
    """Index of the stage whose [start, end) holds `step`; steps at or past the last
    boundary belong to the last stage. `boundaries`: ascending (start, end) pairs."""
    for i, (_, end) in enumerate(boundaries):
        if step < end:
            return i
    return len(boundaries) - 1


def candidate_count(boundaries, step, p_by_stage=None):
    """P for `step` (0 = the full softmax)."""
    table = P_BY_STAGE if p_by_stage is None else p_by_stage
    i = stage_of(boundaries, step)
    counts = table.get(i)
    if not counts:
        return 0
    start, end = boundaries[i]
    part = (step - start) * len(counts) // (end - start)
    return counts[min(max(part, 0), len(counts) - 1)]


def rank_offset(V, rank, world):
    """First sweep index of data-parallel rank `rank` of `world`."""
    if not 0 <= rank < world:
        raise ValueError("rank outside [0, world)")
    return V * rank // world
