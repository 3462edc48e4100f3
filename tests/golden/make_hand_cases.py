"""Write hand_cases.json: small problems whose outputs have closed forms.

The pages print no worked example for the LM-head path, so these fixtures
are closed forms derived by hand (each case states its derivation). The
script uses only the ``math`` module: no oracle, no GPU code.

Softmax cross-entropy over logits z with label t is log(sum_v exp z_v) - z_t
(the textbook definition the chunked backend computes without materialising
the logits; FlashInfer PR #8059, PR description).
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
e = math.e

cases = []

# Case 1: H = I2, W = [[1,0],[0,1],[0,0]] -> z = [[1,0,0],[0,1,0]].
# lse = log(e + 2) on both rows. t = [0, 2]: row losses log(e+2)-1 and log(e+2).
lse = math.log(e + 2.0)
cases.append(dict(
    name="identity_3vocab",
    H=[[1.0, 0.0], [0.0, 1.0]],
    W=[[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]],
    targets=[0, 2],
    derivation="z=[[1,0,0],[0,1,0]]; lse=log(e+2); loss rows lse-1, lse; mean = log(e+2) - 1/2",
    lse=[lse, lse],
    loss_rows=[lse - 1.0, lse],
    loss_mean=lse - 0.5,
    logp=[1.0 - lse, -lse],
    # d loss_mean / dz = (p - onehot)/2, p = [e,1,1]/(e+2) and [1,e,1]/(e+2)
    dz_mean=[[(e / (e + 2) - 1) / 2, (1 / (e + 2)) / 2, (1 / (e + 2)) / 2],
             [(1 / (e + 2)) / 2, (e / (e + 2)) / 2, (1 / (e + 2) - 1) / 2]],
))

# Case 2: one ignored row (-100) and one row with label -5 (every negative label
# is ignored: miles-ext-kernels PR #14, lm_head op commit). Only row 2 counts.
# H rows are multiples of e1; W = [[2,0],[0,0]] -> z row r = [2*h_r0, 0].
cases.append(dict(
    name="negative_labels_ignored",
    H=[[1.0, 0.0], [0.5, 0.0], [0.0, 0.0]],
    W=[[2.0, 0.0], [0.0, 0.0]],
    targets=[-100, -5, 1],
    derivation="only row 2 valid: z=[0,0] -> loss log 2; mean over 1 valid row = log 2",
    lse=[math.log(e ** 2 + 1.0), math.log(e + 1.0), math.log(2.0)],
    loss_rows=[0.0, 0.0, math.log(2.0)],
    loss_mean=math.log(2.0),
    logp=[0.0, 0.0, -math.log(2.0)],
))

# Case 3: support entry, K = 2 candidates [0, 1] over V = 3, logits z = [1, 0, 0]
# lp = z_id - log(e+2); p_hat over {0,1} = [e, 1]/(e+1);
# q = [1/2, 1/2]: KL = sum q (log q - log p_hat) = log(1/2) - (1/2)(log e + log 1) + log(e+1)
cases.append(dict(
    name="support_two_candidates",
    H=[[1.0, 0.0]],
    W=[[1.0, 0.0], [0.0, 1.0], [0.0, 0.0]],
    ids=[[0, 1]],
    ref_logq=[[math.log(0.5), math.log(0.5)]],
    derivation="z=[1,0,0]; lp=[1-log(e+2), -log(e+2)]; KL = log(1/2) - 1/2 + log(e+1)",
    lp=[[1.0 - lse, -lse]],
    kl=[math.log(0.5) - 0.5 + math.log(e + 1.0)],
))

with open(os.path.join(HERE, "hand_cases.json"), "w") as f:
    json.dump(dict(source="hand-derived closed forms; see make_hand_cases.py", cases=cases), f, indent=1)
print("wrote", len(cases), "cases")
