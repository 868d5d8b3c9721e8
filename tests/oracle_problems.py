"""Small decode problems built entirely on the oracle side (numpy + model).

Used by the CPU pins of the oracle and, on the GPU, as the expected side of
parity tests.  Values come from ``workloads`` (seeded), block placement from
``oracle.AllocatorModel`` and cache contents from ``oracle.store_ref``.
"""

import numpy as np

import workloads as W
from oracle import AllocatorModel, store_ref


def model_for(workload, order_seed=None):
    seed = workload.seed if order_seed is None else order_seed
    return AllocatorModel(workload.num_blocks, workload.block_size,
                          workload.max_blocks_per_seq,
                          W.free_order(workload.num_blocks, seed))


def sentinel_caches(workload):
    shape = (workload.num_blocks, workload.block_size, workload.num_kv_heads,
             workload.head_dim)
    kc = W.nan_sentinel_fp16(shape).numpy().view(np.uint16)
    vc = kc.copy()
    return kc, vc


def build_problem(workload, plan_fn=None, alloc=None):
    """Plan with the model, store earlier tokens, then the step's tokens.

    Returns a dict with q, caches before and after the step, tables, lens and
    the step's inputs, all numpy (fp16 arrays as uint16 bit patterns for the
    caches).
    """
    alloc = model_for(workload) if alloc is None else alloc
    plan = (plan_fn or (lambda a: W.plan_for(workload, a)))(alloc)
    hkv, d = workload.num_kv_heads, workload.head_dim
    kc, vc = sentinel_caches(workload)
    slots, idx, distinct = W.prior_scatter(plan)
    if slots:
        kp = W.normal_fp16((len(distinct), hkv, d), W.value_seed(workload, "k_prior")).numpy()
        vp = W.normal_fp16((len(distinct), hkv, d), W.value_seed(workload, "v_prior")).numpy()
        kc, vc = store_ref(kp[idx], vp[idx], slots, kc, vc)
    pre_k, pre_v = kc.copy(), vc.copy()
    B = len(plan.seq_ids)
    k_new = W.normal_fp16((B, hkv, d), W.value_seed(workload, "k_new")).numpy()
    v_new = W.normal_fp16((B, hkv, d), W.value_seed(workload, "v_new")).numpy()
    q = W.normal_fp16((B, workload.num_q_heads, d), W.value_seed(workload, "q")).numpy()
    return {
        "workload": workload,
        "plan": plan,
        "alloc": alloc,
        "q": q,
        "k_new": k_new,
        "v_new": v_new,
        "pre_k": pre_k,
        "pre_v": pre_v,
        "tables": np.asarray(plan.block_tables, dtype=np.int32),
        "lens": np.asarray(plan.context_lens, dtype=np.int32),
        "slots": np.asarray(plan.step_slots, dtype=np.int32),
        "cow_pairs": np.asarray(plan.cow_pairs, dtype=np.int32).reshape(-1, 2),
        "scale": workload.scale,
    }


def after_step(problem):
    """Oracle caches after the step: copy-on-write copies, then the store."""
    from oracle import copy_blocks_ref
    kc, vc = problem["pre_k"], problem["pre_v"]
    if len(problem["cow_pairs"]):
        kc, vc = copy_blocks_ref(kc, vc, problem["cow_pairs"])
    return store_ref(problem["k_new"], problem["v_new"], problem["slots"], kc, vc)
