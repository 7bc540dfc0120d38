"""Mutation check of the oracle's CPU pins (not collected by pytest).

Plants one plausible mistake at a time into a temporary copy of ``oracle/``
(on the CPU only), runs the CPU test suite against the copy and reports every
mutant that no pin catches.  Run:  python tests/oracle_mutation_check.py
"""
import os, shutil, subprocess, sys, tempfile
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTS = [
 ("tiling.py", "u = (dt * ph + dh) * pw + dw", "u = (dh * pt + dt) * pw + dw"),
 ("tiling.py", "j = (it * nH + ih) * nW + iw", "j = (ih * nT + it) * nW + iw"),
 ("tiling.py", "if t < T and h < H and w < W:", "if t < T and h < H and w <= W:"),
 ("estimator.py", "rows.sum(axis=0) / rows.shape[0]", "rows.sum(axis=0) / S"),
 ("estimator.py", "out[j, d:2 * d] = rows.max(axis=0)", "out[j, d:2 * d] = rows.min(axis=0)"),
 ("estimator.py", "out[j, 2 * d:3 * d] = rows.min(axis=0)", "out[j, 2 * d:3 * d] = rows.max(axis=0)"),
 ("estimator.py", "return np.asarray(phi_q, np.float64) @ np.asarray(phi_k, np.float64).T", "return np.asarray(phi_k, np.float64) @ np.asarray(phi_q, np.float64).T"),
 ("estimator.py", "phi = phi + np.asarray(b, np.float64)[None, :]", "phi = phi - np.asarray(b, np.float64)[None, :]"),
 ("select.py", "order = np.lexsort((idx, neg, is_nan))", "order = np.lexsort((-idx, neg, is_nan))"),
 ("select.py", "order = np.lexsort((idx, neg, is_nan))", "order = np.lexsort((idx, neg, ~is_nan))"),
 ("select.py", "return max(1, -(-(n * (100 - s)) // 100))", "return max(1, (n * (100 - s)) // 100)"),
 ("select.py", "col_idx[i * k:(i + 1) * k] = np.sort(order[:k])", "col_idx[i * k:(i + 1) * k] = order[:k]"),
 ("attention.py", "key_slots = key_slots[valid[key_slots]]", "key_slots = key_slots"),
 ("attention.py", "lse = (m + np.log(ssum))[:, 0]", "lse = (np.log(ssum))[:, 0]"),
 ("attention.py", "logits = sm_scale * (q[q_slots] @ k[key_slots].T)", "logits = (q[q_slots] @ k[key_slots].T)"),
 ("attention.py", "kept = col_idx[row_ptr[i]:row_ptr[i + 1]]", "kept = col_idx[row_ptr[i]:row_ptr[i + 1]][:-1] if row_ptr[i+1]-row_ptr[i] > 1 else col_idx[row_ptr[i]:row_ptr[i + 1]]"),
 ("oracle_map.py", "M[a, j] = np.exp(blk - lse[:, None]).max()", "M[a, j] = np.exp(blk - lse[:, None]).mean()"),
 ("oracle_map.py", "cols = cols[valid[cols]]", "cols = cols"),
 ("oracle_map.py", "lse = m + np.log(np.exp(logits - m[:, None]).sum(axis=1))", "lse = m + np.log(np.exp(logits - m[:, None]).sum(axis=1)) + 1e-9"),
 ("oracle_map.py", "all_keys = np.flatnonzero(valid)", "all_keys = np.arange(valid.size)"),
 ("oracle_map.py", "vrows = rows[valid[rows]]", "vrows = rows"),
 ("attention.py", "q_slots = q_slots[valid[q_slots]]", "q_slots = q_slots"),
 ("attention.py", "mask = np.repeat(np.repeat(tile_keep, S, axis=0), S, axis=1)", "mask = np.repeat(np.repeat(tile_keep.T, S, axis=0), S, axis=1)"),
 ("tiling.py", "x[n] = y[s]", "x[n] = y[s] if s % 2 == 0 else 0"),
 ("distill.py", "t * (np.log(safe_t) - log_p)", "np.exp(log_p) * (log_p - np.log(safe_t))"),
 ("distill.py", "g = (p - t) / R", "g = (t - p) / R"),
 ("distill.py", "np.add.at(dphi_q, rows, g @ phi_k)", "dphi_q[rows] = g @ phi_k"),
 ("distill.py", "dphi_k = g.T @ phi_q[rows]", "dphi_k = g.T @ phi_k[rows]"),
 ("distill.py", "dphi_q.sum(axis=0), dphi_k.sum(axis=0)", "dphi_q.sum(axis=0), dphi_q.sum(axis=0)"),
 ("distill.py", "loss = kl_rows(s[rows], map_rows).sum() / R", "loss = kl_rows(s[rows], map_rows).mean()"),
 ("tiling_search.py", "int(np.argmin(errs))", "int(np.argmax(errs))"),
 ("tiling_search.py", "rp, ci = select_topk(s, keep_count(ht.n, sparsity_pct))", "rp, ci = select_topk(s.T, keep_count(ht.n, sparsity_pct))"),
 ("tiling_search.py", "return scatter(np.nan_to_num(o), T, H, W, shape)", "return np.nan_to_num(o)[:T * H * W]"),
 ("tiling_search.py", "full, _ = dense_attention(q, k, v, sm_scale)", "full, _ = dense_attention(q, k, v, 1.0)"),
 ("attention_bwd.py", "ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
 ("attention_bwd.py", "np.add.at(dk, key_slots, sm_scale * ds.T @ q[q_slots])", "dk[key_slots] += sm_scale * ds.T @ q[q_slots]"),
 ("attention_bwd.py", "dq[q_slots] = sm_scale * ds @ k[key_slots]", "dq[q_slots] = ds @ k[key_slots]"),
 ("attention_bwd.py", "np.add.at(dv, key_slots, p.T @ do[q_slots])", "np.add.at(dv, key_slots, ds.T @ do[q_slots])"),
]
env = dict(os.environ)
survivors = []
for f, a, b in MUTS:
    td = tempfile.mkdtemp()
    shutil.copytree(f"{ROOT}/oracle", f"{td}/oracle")
    shutil.copytree(f"{ROOT}/workloads", f"{td}/workloads")
    shutil.copytree(f"{ROOT}/tests", f"{td}/tests")
    p = f"{td}/oracle/{f}"
    s = open(p).read()
    assert a in s, (f, a)
    open(p, "w").write(s.replace(a, b))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", f"{td}/tests"], cwd=td, capture_output=True, text=True)
    killed = r.returncode != 0
    print(("KILLED  " if killed else "SURVIVED"), f, "|", b[:70], flush=True)
    if not killed: survivors.append((f, b))
    shutil.rmtree(td)
print("survivors:", survivors)
sys.exit(1 if survivors else 0)
